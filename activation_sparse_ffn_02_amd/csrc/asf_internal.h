// Internal declarations shared by the host API (asf_api.hip) and the kernels
// (asf_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/asf.h"

namespace asf {

// Workgroups of the fused FFN kernel: one per compute unit of an MI355X.
// Each owns one float32 partial of y, summed by the reduction kernel.
constexpr int kFfnGroups = 256;
constexpr int kFfnThreads = 512;
constexpr int kMaxBatch = 32;
constexpr int kMaxFfn = 65536;  // compaction handles up to 1024 mask words

// Device view of a created layer, carved out of the caller's storage.
struct LayerView {
    int d, f, H, max_batch, gated, wtype;
    float threshold;
    int ws;        // bytes per weight element
    int cd;        // 16-byte chunks per d-long weight row
    int ch;        // 16-byte chunks per H-long weight row
    int words;     // 64-bit mask words: ceil(f / 64)
    int nmat;      // matrices per neuron bundle: 2 (up, down) or 3 (gate, up, down)

    // weights in the library layout
    void *p1;          // [H][d]            predictor layer 1 (as given)
    float *c1;         // [H]
    void *p2;          // [f][H]            predictor layer 2, rows in slot order
    float *c2;         // [f]               slot order
    void *bundles;     // [f][nmat][d]      per slot: (gate,) up row, down column
    float *b1;         // [f]               slot order (gate bias when gated)
    float *b2;         // [d]
    int32_t *perm;     // [f] slot -> original id
    int32_t *inv;      // [f] original id -> slot

    // per-call scratch
    float *h;          // [max_batch][H]
    uint64_t *masks;   // [max_batch][words] per-token masks, slot order
    uint64_t *umask;   // [words] union mask
    int32_t *slots;    // [f] compacted union list, ascending slot
    int32_t *count;    // [1] its length
    float *partial;    // [kFfnGroups][max_batch][d]
    unsigned *bar;     // [2] grid barrier: arrivals, generation
    int *err;          // [1] device error bits (1: a grid barrier wait timed out)
};

size_t carve(const asf_layer_desc &desc, uintptr_t base, LayerView *v);

// ---- launchers (asf_kernels.hip); each returns the hipError_t of its launch
hipError_t launch_perm_rows(const void *src, int chunks_per_row, const int32_t *perm, int nrows,
                            void *dst, size_t dst_stride_chunks, size_t dst_off_chunks,
                            hipStream_t s);
hipError_t launch_transpose_perm(const void *wdown, int d, int f, int ws, const int32_t *inv,
                                 void *bundles, size_t bundle_stride_elems,
                                 size_t dst_off_elems, hipStream_t s);
hipError_t launch_invert(const int32_t *perm, int f, int32_t *inv, hipStream_t s);
hipError_t launch_gather_f32(const float *src, const int32_t *perm, int n, float *dst,
                             hipStream_t s);

// Optional HIP events recorded around each kernel (2 per asf_kernel_id).
struct Trace {
    hipEvent_t ev[2 * ASF_K_COUNT];
};

hipError_t launch_predict(const LayerView &L, const float *x, int B, int32_t *active_ids,
                          int32_t *n_active, uint64_t *token_masks, const Trace *tr,
                          hipStream_t s);

// list_mode: 0 = L.slots/L.count (last prediction), 1 = caller's original ids,
//            2 = every neuron (dense)
hipError_t launch_ffn(const LayerView &L, const float *x, int B, int list_mode,
                      const int32_t *ids, const int32_t *n_ids, const float *resid, float *y,
                      const Trace *tr, hipStream_t s);

// Fused one-launch decode step (B = 1, fp16 weights).
bool fused_supported(const LayerView &L);
hipError_t launch_decode_fused(const LayerView &L, const float *x, const float *resid, float *y,
                               int32_t *active_ids, int32_t *n_active, const Trace *tr,
                               hipStream_t s);
hipError_t launch_read_error(const LayerView &L, int32_t *out, int clear, hipStream_t s);

}  // namespace asf

struct asf_layer {
    asf::LayerView v;
    asf::Trace trace;
    bool tracing;
    bool fused;  // the one-launch decode kernel fits this device and shape
    const asf::Trace *tr() const { return tracing ? &trace : nullptr; }
};
