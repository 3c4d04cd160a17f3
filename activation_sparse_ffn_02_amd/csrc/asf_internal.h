// Internal declarations shared by the host API (asf_api.hip) and the kernels
// (asf_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/asf.h"

namespace asf {

constexpr int kThreads = 512;     // workgroup size of the step kernels (8 waves)
constexpr int kRowsPerWG = 64;    // neuron slots owned by one scoring workgroup
constexpr int kSlices = 16;       // FC2: output slices
constexpr int kGroups = 16;       // FC2: neuron groups (partials per output)
constexpr int kMaxBatch = 32;
constexpr int kPred1MaxB = 4;    // fp16 predictor layer 1 as a GEMV up to this batch, beyond on the matrix cores
constexpr int kMaxFfn = 65536;    // the list kernel handles up to 1024 mask words
constexpr int kArrive = 64;       // arrival counters (FC2 slices, predictor row tiles)
constexpr int kXchCopies = 16;    // copies of h exchanged between the owners (one-launch step)

// k slices of the batched FC1 (1024 k each)
int fc1_slices(int d);
struct LayerView;
// the batched FC2 forms FC1's activations itself (no FC1 finishing kernel);
// all_rows: FC1 ran over every neuron (the dense comparator)
bool fc2_fuses_fin(const LayerView &L, int B, bool all_rows);

// Row pitch (halfs) of the batched form's fp16 copy of x: d rounded up to the
// 512 k that its FC1 takes per stage (the padding stays zero).
inline int x16_pitch(int d) { return (d + 511) / 512 * 512; }

// Chunk i (8 values) of x [B][d] written to x16 as fp16 hi (rows 0 .. Bm-1)
// and lo = the fp16 rounding of what hi left out (rows Bm .. 2Bm-1), pitch dp.
__device__ __forceinline__ void x16_chunk(const float *__restrict__ x, int d, int dp, int Bm,
                                          _Float16 *__restrict__ x16, int i) {
    typedef _Float16 h8v __attribute__((ext_vector_type(8)));
    const int c8 = d / 8, t = i / c8, k = 8 * (i % c8);
    const float4 u = *reinterpret_cast<const float4 *>(x + (size_t)t * d + k);
    const float4 v = *reinterpret_cast<const float4 *>(x + (size_t)t * d + k + 4);
    const float f[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
    h8v hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        hi[e] = (_Float16)f[e];
        lo[e] = (_Float16)(f[e] - (float)hi[e]);
    }
    *reinterpret_cast<h8v *>(x16 + (size_t)t * dp + k) = hi;
    *reinterpret_cast<h8v *>(x16 + (size_t)(Bm + t) * dp + k) = lo;
}

// Position of the r-th set bit of m (r < popcount(m)), by halving.
__device__ __forceinline__ int nth_set_bit(uint64_t m, int r) {
    int pos = 0;
    int c = __popc((uint32_t)m);
    if (r >= c) {
        r -= c;
        m >>= 32;
        pos = 32;
    }
    uint32_t w = (uint32_t)m;
    c = __popc(w & 0xffffu);
    if (r >= c) { r -= c; w >>= 16; pos += 16; }
    c = __popc(w & 0xffu);
    if (r >= c) { r -= c; w >>= 8; pos += 8; }
    c = __popc(w & 0xfu);
    if (r >= c) { r -= c; w >>= 4; pos += 4; }
    c = __popc(w & 0x3u);
    if (r >= c) { r -= c; w >>= 2; pos += 2; }
    if (r >= (int)(w & 1u)) pos += 1;
    return pos;
}

// Device view of a created layer, carved out of the caller's storage.
//
// Neuron work is split over nq = ceil(f / 64) "owner" workgroups: owner q
// holds the slots q, q + nq, q + 2*nq, ... (64 of them, bit i of its mask
// word is slot q + nq*i).  With a hot-first neuron table every owner gets
// the same mix of hot and cold neurons, so per-owner work stays balanced
// without a global prefix sum.
struct LayerView {
    int d, f, H, max_batch, gated, wtype;
    float threshold;
    int ws;        // bytes per weight element
    int cd;        // 16-byte chunks per d-long weight row
    int ch;        // 16-byte chunks per H-long weight row
    int words;     // 64-bit words of a slot-ordered mask: ceil(f / 64)
    int nq;        // owner workgroups (== words)
    int nmat;      // matrices per neuron bundle: 2 (up, down) or 3 (gate, up, down)
    int ncu;       // compute units of the device the layer was created on
    int fused;     // one-token steps run in one launch (every owner resident at once)

    // weights in the library layout
    void *p1;          // [H][d]            predictor layer 1 (as given)
    float *c1;         // [H]
    void *p2;          // [nq*64][H]        predictor layer 2, owner-major: slot q + nq*i
                       //                   at row q*64 + i (rows past f are zero); the
                       //                   batched forms' layout, null when max_batch == 1
    void *p2k;         // [H][nq][64]       the same entries k-major (entry k of slot
                       //                   q + nq*i at (k, q, i)): the one-token form reads
                       //                   the runs of the nonzero h_k
    float *c2;         // [f]               slot order
    void *bundles;     // [f][nmat][d]      per slot: (gate,) up row, down column
    float *b1;         // [f]               slot order (gate bias when gated)
    float *b2;         // [d]
    int32_t *perm;     // [f] slot -> original id
    int32_t *inv;      // [f] original id -> slot

    // per-call scratch
    float *h;          // [max_batch][H]           predictor hidden activations
    _Float16 *h16;     // [2][max_batch][H]        h as fp16 hi, lo (batched form)
    _Float16 *x16;     // [2][max_batch][dp]       x as fp16 hi, lo (batched form;
                       //                          dp = x16_pitch(d), padding zero)
    uint64_t *wbits;   // [max_batch][nq]          per-token owner bits
    uint64_t *ubits;   // [nq]                     union over the batch
    uint64_t *vbits;   // [nq]                     entries listed by each owner
    int32_t *lslot;    // [nq][64]                 their slots (ascending bit); batched
                       //                          form: [rows] in list order
    float *la;         // [nq][64][max_batch]      their FC1 activations
    _Float16 *la16;    // [2][max_batch][nq*64]    batched form: the list rows' FC1
                       //                          activations as fp16 hi, lo, token-major
    float *fc1_part;   // [ks][nmat-1][max_batch][nq*64] batched FC1 partial sums per
                       //                          k slice (ks = fc1_slices(d))
    float *partial;    // [kGroups][max_batch][d]  FC2 partial sums
    float *part1;      // [d/16][nq][16]           single-token FC2 rows per owner
    unsigned *arrive;  // [kArrive]                FC2 arrivals per slice
    float *pred_part;  // [pred_slices(d)][max_batch][H] batched predictor partial sums
    uint64_t *masks;   // [max_batch][words]       slot-ordered token masks
    int32_t *slots;    // [f]                      ascending active slots
    int32_t *count;    // [1]                      their number
    int32_t *rows;     // [1]                      rows of the batched FC1 list
    unsigned *dbg;     // [1]                      debug-build check flags; bit 8: a wait of
                       //                          the one-launch step's h exchange gave up
    uint64_t *xch;     // [kXchCopies][xstride]    h words of the one-launch step
    int xstride;       //                          (epoch << 32 | h bits), H + 64 per copy
    unsigned *epoch;   // [1]                      the step's epoch, advanced by its sum
};

size_t carve(const asf_layer_desc &desc, uintptr_t base, LayerView *v);

// Device view of an attention-head predictor (two-layer X-H-heads MLP).
struct HeadView {
    int d, nh, H, max_batch, wtype;
    float threshold;
    int ws, cd, ch;
    int words;         // 64-bit words of a head mask: ceil(nh / 64)
    void *q1;          // [H][d]
    float *c1;         // [H]
    void *q2;          // [nh][H]
    float *c2;         // [nh]
    float *h;          // [max_batch][H]   scratch: hidden activations
    uint64_t *wbits;   // [max_batch][words] scratch: head words
    _Float16 *h16;     // [2][max_batch][H] scratch of the batched layer 1 (max_batch > 1)
    _Float16 *x16;     // [2][max_batch][x16_pitch(d)]
    float *pred_part;  // [pred_slices(d)][max_batch][H]
    int ncu;           // compute units of the device it was created on
};
constexpr int kMaxHeads = 4096;   // head words per token fit one wave (64)

size_t carve_heads(const asf_head_desc &desc, uintptr_t base, HeadView *v);


// Optional HIP events recorded around each kernel (2 per asf_kernel_id).
struct Trace {
    hipEvent_t ev[2 * ASF_K_COUNT];
};

// ---- create-time layout kernels
// owner_major = nq > 0: slot r = q + nq*i goes to row q*64 + i
hipError_t launch_perm_rows(const void *src, int chunks_per_row, const int32_t *perm, int nrows,
                            void *dst, size_t dst_stride_chunks, size_t dst_off_chunks,
                            int owner_major, hipStream_t s);
hipError_t launch_transpose_perm(const void *wdown, int d, int f, int ws, const int32_t *inv,
                                 void *bundles, size_t bundle_stride_elems,
                                 size_t dst_off_elems, hipStream_t s);
hipError_t launch_invert(const int32_t *perm, int f, int32_t *inv, hipStream_t s);
// P2 [f][H] (original ids) into the k-major layout [H][nq][64]
hipError_t launch_p2_kmajor(const void *p2, int H, int f, int nq, int ws, const int32_t *perm,
                            void *dst, hipStream_t s);
hipError_t launch_gather_f32(const float *src, const int32_t *perm, int n, float *dst,
                             hipStream_t s);

// ---- step kernels
// predictor layer 1: h = ReLU(P1 x + c1)
hipError_t launch_pred_l1(const LayerView &L, const float *x, int B, const Trace *tr,
                          hipStream_t s);
// predictor layer 2 + threshold into owner bits; with fc1, each owner also
// runs FC1 over its union-active neurons (the decode-step form)
hipError_t launch_score(const LayerView &L, const float *x, int B, bool fc1, const Trace *tr,
                        hipStream_t s);
// FC1 over a neuron set without scoring: mode 0 = union of the last
// prediction, 1 = caller's original ids, 2 = every neuron
hipError_t launch_fc1(const LayerView &L, const float *x, int B, int mode, const int32_t *ids,
                      const int32_t *n_ids, const Trace *tr, hipStream_t s);
// FC2 over the owners' lists + per-slice reduction into y; listed: the
// entries' slots come from the list (caller ids) rather than the owner bits;
// all_rows: FC1 ran over every neuron (mode 2)
hipError_t launch_fc2(const LayerView &L, int B, bool listed, const float *resid, float *y,
                      const Trace *tr, hipStream_t s, bool all_rows = false);
// single token, after launch_score with FC1 (or launch_step1): y = sum over
// owners of their FC2 rows (part1) + b2 (+ resid); after launch_step1,
// advance_epoch moves the exchange epoch on for the next step
hipError_t launch_fc2_sum(const LayerView &L, const float *resid, float *y, const Trace *tr,
                          hipStream_t s, bool advance_epoch = false);
// one-token decode step (predict + FC1 + owner FC2 rows) in one launch:
// predictor layer 1 computed by the owners, h exchanged between them through
// memory; needs every owner resident at once (step1_fits, set at create)
bool step1_fits(const LayerView &L);
hipError_t launch_step1(const LayerView &L, const float *x, const Trace *tr, hipStream_t s);
// one token over the set of the last prediction (the owner words), or over
// a caller's list of original ids (ids, n_ids device pointers; ids null =
// the last prediction): FC1 and the owner FC2 rows, as the decode step does
// after its ballot (then launch_fc2_sum)
hipError_t launch_ffn1(const LayerView &L, const float *x, const int32_t *ids,
                       const int32_t *n_ids, const Trace *tr, hipStream_t s);
// one-stream look-ahead stack: layer L's FFN over its set with predictor
// layer 1 of layer N on the same input x, then layer N's scores with layer
// L's owner-row sum (N null: layer L's kernels alone)
hipError_t launch_ffn1_pred1(const LayerView &L, const LayerView *N, const float *x,
                             const Trace *tr, hipStream_t s);
hipError_t launch_score1_fc2sum(const LayerView *N, const LayerView &L, const float *resid,
                                float *y, const Trace *tr, hipStream_t s);
// exact mask, one token: the pre-activation of every neuron, the true set
// (z + b1 > 0) into the owner words, and the owner FC2 rows (then
// launch_fc2_sum)
hipError_t launch_exact1(const LayerView &L, const float *x, bool mask_only, const Trace *tr,
                         hipStream_t s);
// activation profiler: counts[perm[s]] += bit s of the single-token owner
// words (L.wbits); hot-first table by ranking (count desc, id asc)
hipError_t launch_count_bits(const LayerView &L, uint32_t *counts, hipStream_t s);
hipError_t launch_rank_table(const uint32_t *counts, int f, int32_t *table, hipStream_t s);
// batched forms on the matrix cores (B >= 2, fp16 weights)
int pred_slices(int d);   // k slices (512 k) of the batched predictor layer 1
hipError_t launch_pred_mm(const LayerView &L, const float *x, int B, const Trace *tr,
                          hipStream_t s);
hipError_t launch_score_mm(const LayerView &L, int B, const Trace *tr, hipStream_t s);
// x16: take x as fp16 from L.x16 (written by launch_pred_mm for the same x)
hipError_t launch_fc1_mm(const LayerView &L, const float *x, int B, int mode, const int32_t *ids,
                         const int32_t *n_ids, bool x16, const Trace *tr, hipStream_t s);
hipError_t launch_fc2_mm(const LayerView &L, int B, bool all_rows, const float *resid, float *y,
                         const Trace *tr, hipStream_t s);
// attention-head predictor: layer 1 (the FFN predictor's kernels), layer 2 +
// threshold into per-token head words, masks / ascending lists / counts
hipError_t launch_head_predict(const HeadView &V, const float *x, int B, uint64_t *masks,
                               int32_t *heads, int32_t *count, hipStream_t s);
// debug builds: flags |= 1 (id out of range), 2 (id repeated), 4 (count
// outside 0 .. f) for ids[0 .. *n_ids) (n_fixed when n_ids is null), with a
// bitmap of f bits as scratch
hipError_t launch_check_ids(const int32_t *ids, const int32_t *n_ids, int n_fixed, int f,
                            uint32_t *bitmap, unsigned *flags, hipStream_t s);
// slot-ordered outputs of the last prediction: token masks, ascending list
hipError_t launch_list(const LayerView &L, int B, int32_t *active_ids, int32_t *n_active,
                       uint64_t *token_masks, const Trace *tr, hipStream_t s);
// launch_fc2_sum and, in the same grid, the one-token list (ids, count)
hipError_t launch_fc2_sum_list(const LayerView &L, const float *resid, float *y,
                               int32_t *active_ids, int32_t *n_active, const Trace *tr,
                               hipStream_t s, bool advance_epoch);

}  // namespace asf

struct asf_head_predictor {
    asf::HeadView v;
};

struct asf_layer {
    asf::LayerView v;
    asf::Trace trace;
    bool tracing;
    const asf::Trace *tr() const { return tracing ? &trace : nullptr; }
};
