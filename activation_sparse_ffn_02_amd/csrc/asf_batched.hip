// asf_batched.hip -- the batched form (B >= 2 tokens, fp16 weights) of the
// decode step on the matrix cores.  With B tokens sharing one step, every
// weight row the step touches meets all B tokens, so each phase is a skinny
// gathered GEMM: rows x tokens x k.  v_mfma_f32_32x32x16_f16 takes 32 rows x
// 32 tokens x 16 k per instruction (tokens past B are zero and load
// nothing).  Lane layout (gfx950): lane l supplies row (A) / column (B)
// l % 32 with the 8 consecutive k of group l / 32, and accumulator element
// i of lane l holds D[8(i/4) + 4(l/32) + i%4][l % 32].
//
//   predictor layer 1   the FC1 stream below over the rows of P1, x as fp16
//                       hi + lo in LDS (k slices of 512 k); a second kernel
//                       adds the slices' partials, c1, ReLU
//   predictor layer 2   per owner: its 64 slot rows x tokens, k = H; then
//                       threshold and one ballot per token
//   FC1                 the union list spread over row groups x k slices
//                       (1024 k, x slice in LDS), whole-row 1 KiB gathers;
//                       a second kernel adds the slices' partials, then the
//                       activation (small batches on plain layers: the FC2
//                       kernel does that itself)
//   FC2                 tokens x outputs, k = the group's listed neurons;
//                       down segments go through LDS to be read transposed;
//                       a second kernel adds the groups' partials
//
// The predictor feeds x and h to the MFMA as fp16 hi + lo halves (two
// instructions per step), so its sums keep fp32 accuracy and the active
// sets stay those of an fp32 GEMV; FC2 takes the activations as hi + lo
// too; FC1 takes x rounded to fp16 once (an error orders of magnitude inside
// the output tolerance, for half the LDS and operand traffic).
// Every sum runs in a fixed order, so results are reproducible bit for bit.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "asf_internal.h"

namespace asf {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));

constexpr int kW = kThreads / 64;   // waves per workgroup
constexpr int kTile = 32;           // rows / tokens / outputs of one MFMA tile
constexpr int kSliceOut = kTile * kW;  // FC2 outputs per workgroup (256)

__device__ __forceinline__ f32x16 mfma(const h8 a, const h8 b, const f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.0f;
    return z;
}

// row of accumulator element i in lane `lane` (its column is lane % 32)
__device__ __forceinline__ int acc_row(int i, int lane) {
    return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

// Wave tiles -> LDS; returns nothing, caller synchronises.
__device__ __forceinline__ void tile_to_lds(float *dst, const f32x16 &acc, int lane) {
    const int col = lane & 31;
#pragma unroll
    for (int i = 0; i < 16; ++i) dst[acc_row(i, lane) * kTile + col] = acc[i];
}

// ---------------------------------------------------------------- operand tiles through LDS
// Both operands of a 32-row x 32-token x k product stream through LDS in
// chunks of CW 16-byte chunks (8*CW k) per row: the weight tile (32 rows)
// and the token tile (32 token rows of fp16).  Thread t loads chunk t%16
// (and t%16 + 16) of row t/16, so a wave instruction covers 4 rows x 256
// contiguous bytes.  Loads run a few chunks ahead into registers, always
// from clamped addresses and zeroed afterwards (a load under a lane
// condition makes the compiler wait for every outstanding load before the
// next LDS store, which would cancel the prefetch).  A chunk is stored to one
// of two LDS buffers with the 16-byte chunk index XOR-ed with row % 16, so a
// fragment read (32 rows at one chunk) hits distinct banks.  Wave w
// multiplies its CW/16 of the CW/2 MFMA steps of every chunk: a k split over
// the waves, whose 8 partial tiles are added in wave order at the end.
template <int CW> struct Geo {
    static constexpr int LPT = CW / 16;      // loads per thread per tile chunk
    static constexpr int ELEMS = kTile * CW; // 16-byte elements per tile chunk
};

template <int CW> __device__ __forceinline__ int swz(int row, int c) {
    return row * CW + (c ^ (row & 15));
}

__device__ __forceinline__ u32x4 sel4(bool keep, const u32x4 v) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    return keep ? v : z;
}

// this thread's loads of chunk ch of the row at rp (a valid row of C
// chunks), from clamped addresses; the values are zeroed only when stored
// (st_chunk), a ring period later, so that no instruction touches them
// before then
template <int CW>
__device__ __forceinline__ void ld_chunk(const u32x4 *rp, int C, int ch, int lc,
                                         u32x4 (&v)[Geo<CW>::LPT]) {
#pragma unroll
    for (int j = 0; j < Geo<CW>::LPT; ++j) {
        const int c = ch * CW + lc + 16 * j;
        v[j] = rp[c < C ? c : C - 1];
    }
}

// stores chunk ch of this thread's row, zero for chunks past C or a dead row
template <int CW>
__device__ __forceinline__ void st_chunk(u32x4 *buf, int lrow, int lc, bool live, int C, int ch,
                                         const u32x4 (&v)[Geo<CW>::LPT]) {
#pragma unroll
    for (int j = 0; j < Geo<CW>::LPT; ++j) {
        const int c = ch * CW + lc + 16 * j;
        buf[swz<CW>(lrow, lc + 16 * j)] = sel4(live && c < C, v[j]);
    }
}

// fragment of step s of a staged chunk: lane row l%32, k group l/32
template <int CW>
__device__ __forceinline__ h8 frag(const u32x4 *buf, int s, int lane) {
    return __builtin_bit_cast(h8, buf[swz<CW>(lane & 31, 2 * s + (lane >> 5))]);
}

// The 8 wave partial tiles (red[w*1024 + row*32 + col]) summed in wave
// order; thread tid owns elements tid and tid + 512.
__device__ __forceinline__ void tile_sum(const float *red, float (&v)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int e = threadIdx.x + kThreads * j;
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < kW; ++w) sum += red[w * kTile * kTile + e];
        v[j] = sum;
    }
}

// ---------------------------------------------------------------- predictor layer 2
// Owner q: rows i = 0..63 (slot q + nq*i) in two 32-row tiles, each streamed
// with the token tiles of h (fp16 hi and lo, two MFMAs per step) over k = H in
// chunks of 128 k.  Scores = tile sums + c2; wave w ballots tokens w, w+8, ...
// into the per-token owner words; the union is their OR.
__global__ __launch_bounds__(kThreads) void k_score_mm(const u32x4 *__restrict__ P2,
                                                       const float *__restrict__ c2,
                                                       const _Float16 *__restrict__ h16, int B,
                                                       int H, int f, float theta,
                                                       uint64_t *__restrict__ wbits,
                                                       uint64_t *__restrict__ ubits) {
    constexpr int CW = 16;
    constexpr int EL = Geo<CW>::ELEMS;
    constexpr int PRE = 2;                           // chunk stages in flight per thread
    __shared__ u32x4 smem[2 * 4 * EL];               // [buffer][A0, A1, h hi, h lo] chunks; later the wave tiles
    __shared__ float sc[2 * kTile][kTile + 1];
    __shared__ uint64_t uw[kW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q = blockIdx.x, nq = gridDim.x;
    const int C = H / 8;
    const int nch = (C + CW - 1) / CW;
    const int lrow = tid / 16, lc = tid % 16;
    const u32x4 *rp[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) rp[t] = P2 + (size_t)(q * kRowsPerWG + kTile * t + lrow) * C;   // owner-major rows
    const bool tokr = lrow < B;
    const u32x4 *hhi = reinterpret_cast<const u32x4 *>(h16 + (size_t)(tokr ? lrow : 0) * H);
    const u32x4 *hlo = reinterpret_cast<const u32x4 *>(h16 + (size_t)(B + (tokr ? lrow : 0)) * H);
    // a chunk stage carries both row tiles of the owner and the h chunk they
    // share; stages past nch load clamped and store zeros (the loop body stays
    // free of branches, so the ring registers carry over without copies that
    // would wait)
    u32x4 ra[PRE][4][1];
    auto load = [&](int ch, u32x4 (&v)[4][1]) {
        ld_chunk<CW>(rp[0], C, ch, lc, v[0]);
        ld_chunk<CW>(rp[1], C, ch, lc, v[1]);
        ld_chunk<CW>(hhi, C, ch, lc, v[2]);
        ld_chunk<CW>(hlo, C, ch, lc, v[3]);
    };
#pragma unroll
    for (int u = 0; u < PRE; ++u) load(u, ra[u]);
    f32x16 acc0 = zero16(), acc1 = zero16();
    auto pass = [&](int ch0) {
#pragma unroll
        for (int u = 0; u < PRE; ++u) {
            const int ch = ch0 + u;
            u32x4 *bufp = smem + (u & 1) * 4 * EL;     // consecutive stages alternate buffers
            st_chunk<CW>(bufp, lrow, lc, true, C, ch, ra[u][0]);
            st_chunk<CW>(bufp + EL, lrow, lc, true, C, ch, ra[u][1]);
            st_chunk<CW>(bufp + 2 * EL, lrow, lc, tokr, C, ch, ra[u][2]);
            st_chunk<CW>(bufp + 3 * EL, lrow, lc, tokr, C, ch, ra[u][3]);
            load(ch + PRE, ra[u]);
            __syncthreads();
            const h8 a0 = frag<CW>(bufp, wave, lane);
            const h8 a1 = frag<CW>(bufp + EL, wave, lane);
            const h8 bh = frag<CW>(bufp + 2 * EL, wave, lane);
            const h8 bl = frag<CW>(bufp + 3 * EL, wave, lane);
            acc0 = mfma(a0, bh, acc0);
            acc0 = mfma(a0, bl, acc0);
            acc1 = mfma(a1, bh, acc1);
            acc1 = mfma(a1, bl, acc1);
        }
    };
    // first pass peeled: the loop is entered from a copy of its body, so the
    // wait at its head need not cover every load in flight
    pass(0);
    for (int ch0 = PRE; ch0 < nch; ch0 += PRE) pass(ch0);
    // tile sums -> sc[i][t]
    float *red = reinterpret_cast<float *>(smem);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        __syncthreads();
        tile_to_lds(red + wave * kTile * kTile, t == 0 ? acc0 : acc1, lane);
        __syncthreads();
        float v[2];
        tile_sum(red, v);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int e = tid + kThreads * j;
            sc[kTile * t + e / kTile][e % kTile] = v[j];
        }
    }
    __syncthreads();
    const int i = lane;
    const int slot_i = q + nq * i;
    const bool valid_i = slot_i < f;
    const float bias = c2[valid_i ? slot_i : f - 1];
    uint64_t u = 0;
    for (int t = wave; t < B; t += kW) {
        const uint64_t m = __ballot(valid_i && sc[i][t] + bias > theta);
        if (lane == 0) wbits[(size_t)t * nq + q] = m;
        u |= m;
    }
    if (lane == 0) uw[wave] = u;
    __syncthreads();
    if (tid == 0) {
        uint64_t all = 0;
#pragma unroll
        for (int w = 0; w < kW; ++w) all |= uw[w];
        ubits[q] = all;
    }
}

// ---------------------------------------------------------------- buffer loads
// Raw buffer loads: the resource bounds the access to [base, base + bytes);
// a 16-byte load at an offset past the bound returns zeros without a memory
// access, so loads of absent rows or tokens are issued like any other (the
// count in flight does not depend on data and the compiler's waits stay
// exact).  Base and bound must be wave-uniform.  Every weight array fits 32-bit
// offsets (at most 65536 bundles of 3 x 16 KiB).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kBufWord3 = 0x00020000;     // descriptor word 3: 32-bit data format
constexpr uint32_t kOob = 0xFFFFFFF0u;    // an offset past every bound

__device__ __forceinline__ rsrc_t buf_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kBufWord3);
}
// weights: streamed once (non-temporal)
__device__ __forceinline__ u32x4 ld_stream(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
}
// operands every workgroup reads (x, activations): cached
__device__ __forceinline__ u32x4 ld_shared(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// ---------------------------------------------------------------- FC1
struct Fc1MmParams {
    const void *bundles;
    uint32_t bundle_bytes;   // bytes per bundle
    uint32_t all_bytes;      // f bundles
    int cd;                  // chunks per d row
    const float *b1;
    const _Float16 *x16;     // [2][Bm][dp] x as fp16 hi, lo (padding zero); FC1 reads hi
    int dp, Bm;
    int B, f, nq;
    int mode;                // 0 union of the last prediction, 1 caller ids, 2 all
    const uint64_t *ubits;
    const int32_t *ids;
    const int32_t *n_ids;
    const int32_t *inv;
    int32_t *lslot;          // [rows] slot of list row r (-1: a skipped caller id)
    _Float16 *la16;          // [2][Bm][LR] activations hi, lo, token-major
    int LR;
    int32_t *rows;           // number of list rows
    float *part;             // [ks][NM][Bm][LR] partial sums per k slice
    int ks;                  // k slices
    int add_b1;              // slice 0 adds b1 (b1 is read, and stays valid, either way)
};

// x -> fp16 hi + lo (for FC1 calls that follow no predictor pass)
__global__ void k_to_f16(const float *__restrict__ x, int B, int d, int dp, int Bm,
                         _Float16 *__restrict__ x16) {
    const int n8 = B * d / 8;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += gridDim.x * blockDim.x)
        x16_chunk(x, d, dp, Bm, x16, i);
}

// The FC1 list: mode 0 the union of the last prediction, owner by owner
// (row r is the (r - pre[q])-th set bit i of owner q, slot q + nq*i, for the
// owner with pre[q] <= r < pre[q+1], pre the popcount prefix); mode 1 the
// caller's ids in list order; mode 2 every slot.
//
// Workgroup (g, ks) takes the list rows of group g (the list spread evenly
// over GR groups) over the k slice ks (1024 k; KS slices cover d): its slice
// of x (32 tokens x 1024 k as fp16, 64 KiB) is read once into LDS, so the
// weight stream carries no x traffic, and the KS partial sums of a row are
// added by k_fc1_fin.  The rows go in passes of NRT row tiles (32 rows);
// a stage is one row tile x one 1 KiB piece (512 k) of one matrix: each
// piece of a row is one buffer load of one wave, so every request reads a
// row contiguously (the gather pattern that streams fastest; absent rows and
// pieces past d read nothing), kFc1Pre stages ahead, also across passes.
// The stage goes through LDS (16-byte chunks XOR-swizzled by row) to be read
// as MFMA fragments; wave w takes chunks 8w .. 8w+7 of the piece, its lane
// (row or token t, half h) the k groups of chunks 8w+4h .. 8w+4h+3 on both
// sides.  At the end of a pass each row tile's eight wave tiles are added in
// wave order into the partial sums.
constexpr int kPieceK = 512;                   // k per row piece (1 KiB of fp16)
constexpr int kPieceC = kPieceK / 8;           // 16-byte chunks per piece (64)
constexpr int kSliceP = 2;                     // pieces per k slice
constexpr int kSliceC = kSliceP * kPieceC;     // chunks per token row of the x slice (128)
constexpr int kStageCh = kTile * kPieceC;      // chunks per stage buffer (32 KiB)
constexpr int kFc1Pre = 4;                     // stages in flight
constexpr int kFc1MaxRows = 2048;              // rows per workgroup (the grid guarantees it)
constexpr int kMaxKSlices = 8;                 // d <= 8192
constexpr int kMaxPredSlices = 16;             // predictor slices of 512 k, d <= 8192

// HILO: x as fp16 hi + lo (two MFMAs per k-step) in slices of one piece (the
// LDS holds hi and lo of 512 k), as the batched predictor layer 1 takes it
template <bool GATED, int NRT_, bool HILO = false> struct Fc1Geo {
    static constexpr int NM = GATED ? 2 : 1;               // matrices per row: [gate,] up
    static constexpr int NRT = NRT_;                       // row tiles per pass
    static constexpr int SP = HILO ? 1 : kSliceP;          // pieces per k slice
    static constexpr int XC = SP * kPieceC;                // chunks per token row of a half of xs
    static constexpr int SPP = NRT * SP * NM;              // stages per pass
    static constexpr int PRE = SPP < kFc1Pre ? SPP : kFc1Pre;  // stages in flight
    static_assert(SPP % PRE == 0 && PRE % 2 == 0, "ring slots repeat every pass");
    static_assert(XC * (HILO ? 2 : 1) == kSliceC, "the x slice fills its LDS");
};

// wave tile -> LDS, element (row, col) at row*32 + (col ^ row), so that both
// the rows of a column (the epilogue's reads) and the columns of a row (the
// writes) fall on distinct banks
__device__ __forceinline__ void tile_to_lds_x(float *dst, const f32x16 &acc, int lane) {
    const int col = lane & 31;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int row = acc_row(i, lane);
        dst[row * kTile + (col ^ row)] = acc[i];
    }
}

struct NoHook {
    __device__ void operator()() const {}
};

// The weight stream of workgroup slice ks over its nr rows (slots in rslot,
// x slice in xs), in passes of NRT row tiles.  `hook` runs once the first
// stages are requested and before their first barrier: a caller whose x
// slice is still in flight stores it to xs there.
template <bool GATED, int NRT, bool HILO = false, class Hook = NoHook>
__device__ __forceinline__ void fc1_stream(const Fc1MmParams &p, const u32x4 *xs, u32x4 *stg,
                                           const int *rslot, int ks, int r0, int nr,
                                           Hook hook = {}) {
    using G1 = Fc1Geo<GATED, NRT, HILO>;
    constexpr int NM = G1::NM, SPP = G1::SPP, SP = G1::SP, XC = G1::XC, PRE = G1::PRE;
    constexpr int TT = kTile * kTile;
    static_assert((NRT * NM) % 2 == 0 && 2 * kW * TT * 4 <= 2 * kStageCh * 16,
                  "the epilogue reduces two tiles per round in the stage buffers");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // ---- the weight stream
    const int npass = (nr + kTile * NRT - 1) / (kTile * NRT);
    const uint32_t rowb = 16u * (uint32_t)p.cd;                // bytes of a weight row
    const int tk = lane & 31, hh = lane >> 5;
    // stage j of pass ps: row tile j / (2 NM), piece (j / NM) % 2, matrix j % NM;
    // wave w loads rows w, w+8, w+16, w+24 of the tile
    auto issue = [&](int ps, int j, u32x4 (&w)[4]) {
        const int i = j / (SP * NM), pc = (j / NM) % SP, m = j % NM;
        const uint32_t koff = 1024u * (uint32_t)(SP * ks + pc);
        const uint32_t moff = (GATED && m == 1) ? rowb : 0u;   // [gate,] up
        // the four slots read together (clamped index, unconditional)
        int sv[4];
#pragma unroll
        for (int l = 0; l < 4; ++l) {
            const int rr = kTile * (NRT * ps + i) + wave + kW * l;
            sv[l] = rslot[rr < kFc1MaxRows ? rr : kFc1MaxRows - 1];
        }
#pragma unroll
        for (int l = 0; l < 4; ++l) {
            const int rr = kTile * (NRT * ps + i) + wave + kW * l;
            const int sl = __builtin_amdgcn_readfirstlane(rr < nr ? sv[l] : -1);
            const bool ok = sl >= 0 && koff < rowb;
            const char *base = static_cast<const char *>(p.bundles) +
                               (ok ? (size_t)sl * p.bundle_bytes + moff + koff : 0);
            w[l] = ld_stream(buf_rsrc(base, ok ? rowb - koff : 0u), 16u * lane);
        }
    };
    u32x4 ring[PRE][4];
#pragma unroll
    for (int u = 0; u < PRE; ++u) issue(0, u, ring[u]);
    hook();
    f32x16 acc[NRT * NM];
    float *red = reinterpret_cast<float *>(stg);
    auto pass = [&](int ps) {
#pragma unroll
        for (int a = 0; a < NRT * NM; ++a) acc[a] = zero16();
        // slice 0 adds b1 to the (gate or up) sum of a present row: the b1 of
        // this thread's epilogue rows, requested before the pass's stages
        // (every slice loads, from a clamped index, and keeps zero)
        float bias[NRT * NM / 2][4];
#pragma unroll
        for (int a0 = 0; a0 < NRT * NM; a0 += 2)
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const int e = tid + kThreads * h;
                const int a = a0 + e / TT, i = a / NM, rr = e % kTile;
                const int row = kTile * (NRT * ps + i) + rr;
                const int sl = rslot[row < nr ? row : 0];
                const bool use = p.add_b1 && ks == 0 && row < nr && sl >= 0;
                const float b = p.b1[use ? sl : 0];
                bias[a0 / 2][h] = use ? b : 0.0f;
            }
#pragma unroll
        for (int j = 0; j < SPP; ++j) {
            const int u = j % PRE, b = j & 1;
            const int i = j / (SP * NM), pc = (j / NM) % SP, m = j % NM;
            u32x4 *bufp = stg + b * kStageCh;
#pragma unroll
            for (int l = 0; l < 4; ++l) {
                const int row = wave + kW * l;
                bufp[row * kPieceC + (lane ^ (row & 15))] = ring[u][l];
            }
            if (j + PRE < SPP) issue(ps, j + PRE, ring[u]);
            else issue(ps + 1, j + PRE - SPP, ring[u]);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int c = 8 * wave + 4 * hh + kk;
                const h8 a = __builtin_bit_cast(h8, bufp[tk * kPieceC + (c ^ (tk & 15))]);
                const int cx = kPieceC * pc + c;
                const h8 bx = __builtin_bit_cast(h8, xs[tk * XC + (cx ^ (tk & 15))]);
                acc[i * NM + m] = mfma(a, bx, acc[i * NM + m]);
                if constexpr (HILO) {
                    const h8 bl = __builtin_bit_cast(h8, xs[(kTile + tk) * XC + (cx ^ (tk & 15))]);
                    acc[i * NM + m] = mfma(a, bl, acc[i * NM + m]);
                }
            }
        }
        // pass end: each row tile's wave tiles summed in wave order into the
        // partial sums of this slice (two tiles per round), rows fastest
        // (coalesced stores)
#pragma unroll
        for (int a0 = 0; a0 < NRT * NM; a0 += 2) {
            __syncthreads();
            tile_to_lds_x(red + wave * TT, acc[a0], lane);
            tile_to_lds_x(red + (kW + wave) * TT, acc[a0 + 1], lane);
            __syncthreads();
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const int e = tid + kThreads * h;
                const int a = a0 + e / TT, i = a / NM, m = a % NM;
                const int t = (e % TT) / kTile, rr = e % kTile;
                const int row = kTile * (NRT * ps + i) + rr;
                float sum = 0.0f;
#pragma unroll
                for (int w = 0; w < kW; ++w)
                    sum += red[((e / TT) * kW + w) * TT + rr * kTile + (t ^ rr)];
                if (m == 0) sum += bias[a0 / 2][h];
                if (t < p.B && row < nr)
                    p.part[((size_t)(ks * NM + m) * p.Bm + t) * p.LR + r0 + row] = sum;
            }
        }
        __syncthreads();
    };
    // the first pass is peeled: the loop is then entered from a copy of its
    // own body (partial stores included), so the wait at its head stays
    // fine-grained
    pass(0);
    for (int ps = 1; ps < npass; ++ps) pass(ps);
}

template <bool GATED>
__global__ __launch_bounds__(kThreads) void k_fc1_mm(Fc1MmParams p) {
    __shared__ u32x4 xs[kTile * kSliceC];            // x slice [token][chunk], swizzled
    __shared__ u32x4 stg[2 * kStageCh];              // stage buffers; before: owner words; pass ends: wave tiles
    __shared__ int pre[kMaxFfn / 64 + 1];
    __shared__ int rslot[kFc1MaxRows];
    __shared__ int wave_tot[kW];
    __shared__ int nrows_lds;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int KS = p.ks, ks = blockIdx.x % KS, g = blockIdx.x / KS, GR = gridDim.x / KS;
    // ---- this slice of x, requested first (tokens past B read zeros; a slice
    // past d reads x of the next token or zeros: finite, against zero weights)
    const int xt = tid >> 4, xc = tid & 15;
    u32x4 xv[kSliceC / 16];
    {
        const rsrc_t xh = buf_rsrc(p.x16, (uint32_t)p.B * p.dp * 2);
        const uint32_t xo = (uint32_t)(xt * p.dp + kSliceP * kPieceK * ks) * 2;
#pragma unroll
        for (int j = 0; j < kSliceC / 16; ++j) xv[j] = ld_shared(xh, xo + 16u * (xc + 16 * j));
    }
    // ---- the list's length
    const uint64_t *vb = reinterpret_cast<const uint64_t *>(stg);
    if (p.mode == 0) {
        uint64_t *vw = reinterpret_cast<uint64_t *>(stg);
        const int nq = p.nq;
        for (int q = tid; q < nq; q += kThreads) vw[q] = p.ubits[q];
        __syncthreads();
        const int q0 = 2 * tid, q1 = 2 * tid + 1;
        const int c0 = q0 < nq ? __popcll(vb[q0]) : 0, c1 = q1 < nq ? __popcll(vb[q1]) : 0;
        const int sum = c0 + c1;
        int incl = sum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(incl, o, 64);
            if (lane >= o) incl += v;
        }
        if (lane == 63) wave_tot[wave] = incl;
        __syncthreads();
        int base = 0;
        for (int w = 0; w < wave; ++w) base += wave_tot[w];
        const int excl = base + incl - sum;
        if (q0 < nq) pre[q0] = excl;
        if (q1 < nq) pre[q1] = excl + c0;
        if (tid == kThreads - 1) {
            pre[nq] = base + incl;
            nrows_lds = base + incl;
        }
    } else if (tid == 0) {
        int n = p.f;
        if (p.mode == 1) {
            n = *p.n_ids;
            n = n < 0 ? 0 : (n > p.f ? p.f : n);
        }
        nrows_lds = n;
    }
    __syncthreads();
    const int nrows = nrows_lds;
    const int R = (nrows + GR - 1) / GR;
    const int r0 = R * g;
    if (r0 >= nrows) {
        if (blockIdx.x == 0 && tid == 0) *p.rows = nrows;
        return;
    }
    const int nr = R < nrows - r0 ? R : nrows - r0;
    // ---- this workgroup's slots; x slice to LDS
    for (int i = tid; i < nr; i += kThreads) {
        const int r = r0 + i;
        int slot;
        if (p.mode == 0) {
            int lo = 0, hi = p.nq;                   // largest q with pre[q] <= r
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (pre[mid] <= r) lo = mid;
                else hi = mid;
            }
            slot = lo + p.nq * nth_set_bit(vb[lo], r - pre[lo]);
        } else if (p.mode == 2) {
            slot = r;
        } else {
            const int id = p.ids[r];
            slot = (unsigned)id < (unsigned)p.f ? p.inv[id] : -1;
            if ((unsigned)slot >= (unsigned)p.f) slot = -1;
        }
        rslot[i] = slot;
        if (ks == 0) p.lslot[r] = slot;
    }
#pragma unroll
    for (int j = 0; j < kSliceC / 16; ++j) {
        const int c = xc + 16 * j;
        xs[xt * kSliceC + (c ^ (xt & 15))] = xv[j];
    }
    __syncthreads();
    // ---- the weight stream, passes sized to the rows (wave-uniform)
    if constexpr (GATED) {
        if (nr <= kTile) fc1_stream<true, 1>(p, xs, stg, rslot, ks, r0, nr);
        else if (nr <= 2 * kTile) fc1_stream<true, 2>(p, xs, stg, rslot, ks, r0, nr);
        else fc1_stream<true, 3>(p, xs, stg, rslot, ks, r0, nr);
    } else {
        if (nr <= 2 * kTile) fc1_stream<false, 2>(p, xs, stg, rslot, ks, r0, nr);
        else if (nr <= 4 * kTile) fc1_stream<false, 4>(p, xs, stg, rslot, ks, r0, nr);
        else fc1_stream<false, 6>(p, xs, stg, rslot, ks, r0, nr);
    }
    if (blockIdx.x == 0 && tid == 0) *p.rows = nrows;
}

// The KS partial sums of each list row and token added in slice order (slice
// 0 carries b1), then the activation: a = ReLU(up . x + b1) (gated:
// ReLU(gate . x + b1) * (up . x)), written as fp16 hi + lo to la16
// (token-major).  A row whose caller id was skipped has zero sums.  Thread:
// token t, rows 8c .. 8c+7, its loads issued beside the list length; rows
// past the list (up to the next multiple of 8, which FC2 reads in 8-row
// chunks) get zeros.
template <bool GATED>
__global__ __launch_bounds__(256) void k_fc1_fin(Fc1MmParams p) {
    constexpr int NM = GATED ? 2 : 1;
    const int c8 = p.LR / 8;
    const int gid = blockIdx.x * 256 + threadIdx.x;
    if (gid >= p.B * c8) return;
    const int t = gid / c8, r = 8 * (gid % c8);
    const int KS = p.ks;
    const int n = *p.rows;
    // every slice's loads in flight (unrolled to the largest count, clamped)
    float4 v[kMaxKSlices][NM][2];
#pragma unroll
    for (int s = 0; s < kMaxKSlices; ++s)
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const float *q = p.part + ((size_t)((s < KS ? s : 0) * NM + m) * p.Bm + t) * p.LR + r;
            v[s][m][0] = *reinterpret_cast<const float4 *>(q);
            v[s][m][1] = *reinterpret_cast<const float4 *>(q + 4);
        }
    if (r >= n) return;
    float sum[NM][8];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) sum[m][e] = 0.0f;
#pragma unroll
    for (int s = 0; s < kMaxKSlices; ++s) {
        if (s < KS) {
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const float f[8] = {v[s][m][0].x, v[s][m][0].y, v[s][m][0].z, v[s][m][0].w,
                                    v[s][m][1].x, v[s][m][1].y, v[s][m][1].z, v[s][m][1].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) sum[m][e] += f[e];
            }
        }
    }
    h8 hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float a = 0.0f;
        if (r + e < n) {
            if constexpr (GATED) a = fmaxf(sum[0][e], 0.0f) * sum[1][e];
            else a = fmaxf(sum[0][e], 0.0f);
        }
        hi[e] = (_Float16)a;
        lo[e] = (_Float16)(a - (float)hi[e]);
    }
    *reinterpret_cast<h8 *>(p.la16 + (size_t)t * p.LR + r) = hi;
    *reinterpret_cast<h8 *>(p.la16 + (size_t)(p.Bm + t) * p.LR + r) = lo;
}

// ---------------------------------------------------------------- predictor layer 1 (stream form)
// Batched predictor layer 1 on the FC1 stream: workgroup (g, ks) takes the
// P1 rows of group g over k slice ks (512 k), x read once as fp32 and kept
// in LDS as fp16 hi + lo (two MFMAs per k-step, so the sums keep fp32
// accuracy and the active sets stay those of an fp32 GEMV); the KS partial
// sums of each row and token go to k_pred_sum.
__global__ __launch_bounds__(kThreads) void k_pred_rows(Fc1MmParams p, const float *__restrict__ x,
                                                        int d) {
    __shared__ u32x4 xs[kTile * kSliceC];            // [hi rows 0-31 | lo rows 32-63][64 chunks]
    __shared__ u32x4 stg[2 * kStageCh];
    __shared__ int rslot[kFc1MaxRows];
    const int tid = threadIdx.x;
    const int KS = p.ks, ks = blockIdx.x % KS, g = blockIdx.x / KS, GR = gridDim.x / KS;
    // x slice: token xt, chunks xc + 16j (8 k each); tokens past B read zeros,
    // k past d reads x of the next token (against zero weights) or zeros
    const int xt = tid >> 4, xc = tid & 15;
    const rsrc_t xr = buf_rsrc(x, (uint32_t)p.B * d * 4);
    u32x4 v[kPieceC / 16][2];
#pragma unroll
    for (int j = 0; j < kPieceC / 16; ++j) {
        const uint32_t o = (uint32_t)(xt * d + kPieceK * ks + 8 * (xc + 16 * j)) * 4;
        v[j][0] = ld_shared(xr, o);
        v[j][1] = ld_shared(xr, o + 16);
    }
    // x as hi + lo into LDS, run by the stream once its first stages are
    // requested (the x loads were issued first, so waiting for them does not
    // wait for the weights)
    auto store_x = [&]() {
#pragma unroll
        for (int j = 0; j < kPieceC / 16; ++j) {
            const int c = xc + 16 * j;
            const float4 u0 = __builtin_bit_cast(float4, v[j][0]);
            const float4 u1 = __builtin_bit_cast(float4, v[j][1]);
            const float fv[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
            h8 hi, lo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                hi[e] = (_Float16)fv[e];
                lo[e] = (_Float16)(fv[e] - (float)hi[e]);
            }
            xs[xt * kPieceC + (c ^ (xt & 15))] = __builtin_bit_cast(u32x4, hi);
            xs[(kTile + xt) * kPieceC + (c ^ (xt & 15))] = __builtin_bit_cast(u32x4, lo);
        }
    };
    const int H = p.f;
    const int R = (H + GR - 1) / GR;
    const int r0 = R * g;
    const int nr = r0 < H ? (R < H - r0 ? R : H - r0) : 0;
    for (int i = tid; i < nr; i += kThreads) rslot[i] = r0 + i;
    __syncthreads();
    if (nr <= 0) return;
    if (nr <= 2 * kTile) fc1_stream<false, 2, true>(p, xs, stg, rslot, ks, r0, nr, store_x);
    else fc1_stream<false, 4, true>(p, xs, stg, rslot, ks, r0, nr, store_x);
}

// Element (t, r): the KS partial sums of row r for token t in slice order,
// then c1, then ReLU -> h and its fp16 hi/lo halves.  The grid also converts
// x to fp16 hi + lo for the FC1 of the step.
__global__ __launch_bounds__(kThreads) void k_pred_sum(const float *__restrict__ part, int KS,
                                                       int Bm, const float *__restrict__ c1,
                                                       const float *__restrict__ x, int B, int d,
                                                       int H, float *__restrict__ h,
                                                       _Float16 *__restrict__ h16,
                                                       _Float16 *__restrict__ x16, int dp) {
    const int gid = blockIdx.x * kThreads + threadIdx.x;
    if (gid < B * H) {
        const int t = gid / H, r = gid % H;
        // every slice's load in flight (unrolled to the largest count, clamped)
        float pv[kMaxPredSlices];
#pragma unroll
        for (int s = 0; s < kMaxPredSlices; ++s)
            pv[s] = part[((size_t)(s < KS ? s : 0) * Bm + t) * H + r];
        float sum = 0.0f;
#pragma unroll
        for (int s = 0; s < kMaxPredSlices; ++s)
            if (s < KS) sum += pv[s];
        const float hv = fmaxf(sum + c1[r], 0.0f);
        const _Float16 hi = (_Float16)hv;
        h[(size_t)t * H + r] = hv;
        h16[(size_t)t * H + r] = hi;
        h16[(size_t)(B + t) * H + r] = (_Float16)(hv - (float)hi);
    }
    const int n8 = B * d / 8;
    for (int i = gid; i < n8; i += gridDim.x * kThreads) x16_chunk(x, d, dp, Bm, x16, i);
}

// ---------------------------------------------------------------- FC2
struct Fc2MmParams {
    const void *bundles;
    uint32_t bundle_bytes;   // bytes per bundle
    uint32_t all_bytes;      // f bundles
    uint32_t dn_off;         // byte offset of the down column in a bundle
    int cd;                  // chunks per down column
    const int32_t *lslot;
    const _Float16 *la16;    // [2][Bm][LR]
    int LR, Bm;
    const int32_t *rows;
    int d, B;
    float *partial;          // [groups][B][d]
    int groups;              // list-row ranges (<= kGroups)
    const float *part;       // FUSED: FC1's k-slice partials [ks][1][Bm][LR]
    int ks;                  // FUSED: k slices (<= kFc2FuseKS)
};

constexpr int kFc2N = 64;                   // list rows per step (4 MFMA k-steps)
constexpr int kWPitch = kSliceOut + 8;      // halfs per staged down row
constexpr int kAPitch = kFc2N + 8;          // halfs per staged token row of a
constexpr int kFc2Pre = 4;                  // steps in flight
constexpr int kFc2Rows = 8192;              // list rows per group (f <= 65536, >= 8 groups)
constexpr int kFc2FuseKS = 5;               // FUSED: at most this many FC1 k slices (d <= 5120)

// 16-byte chunk of staged down row r holding outputs 8c .. 8c+7: rows 32
// apart sit 4 chunks apart, so the two half-waves of a fragment read (rows
// r and r + 32, the same 32 outputs) use different banks
__device__ __forceinline__ int wl_chunk(int r, int c) { return c ^ (((r >> 5) & 1) << 2); }

// Workgroup (slice s, group g): outputs 256s .. 256s+255 over the list rows
// of steps [S*g/G, S*(g+1)/G) (S steps of 64 rows).  Per step each thread
// loads four 16-byte chunks of down columns (rows tid/32 + 16j, chunk tid%32
// of the slice: two rows x 512 contiguous bytes per wave load; absent rows
// and chunks read nothing) and one chunk of a (hi or lo half, token, 8 rows),
// four steps ahead; the step goes through LDS (double buffered) and wave w
// multiplies tokens x its 32 outputs x 64 rows, a as hi + lo (two MFMAs per
// k-step), the down fragments read transposed.  Rows are paired with the
// same permutation on both sides: lane half h takes rows 32h + 8j .. 32h+8j+7
// at k-step j.  Group tiles go to `partial`; k_fc2_fin adds the G in group
// order, then b2, then the residual.
//
// FUSED (plain layers of at most kFc2FuseKS FC1 k slices, small batches): a
// is formed here from FC1's k-slice partials instead of read from la16, so
// FC1 needs no finishing kernel: thread t takes token t / 16 and rows
// 4 (t % 16) .. +3 of the step, sums its KS partials in slice order, applies
// the ReLU (rows past the list are zero) and splits the result into fp16 hi
// + lo, exactly as k_fc1_fin does.
template <bool FUSED>
__global__ __launch_bounds__(kThreads) void k_fc2_mm(Fc2MmParams p) {
    __shared__ __attribute__((aligned(16))) _Float16 wl[2][kFc2N * kWPitch];
    __shared__ __attribute__((aligned(16))) _Float16 al[2][2 * kTile * kAPitch];
    __shared__ int rslot[kFc2Rows];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = p.groups;
    const int nslice = gridDim.x / G;
    const int s = blockIdx.x % nslice, g = blockIdx.x / nslice;
    const int R = *p.rows;
    const int S = (R + kFc2N - 1) / kFc2N;
    const int sb = (int)((long long)S * g / G), se = (int)((long long)S * (g + 1) / G);
    const int rb = kFc2N * sb;
    const int re = kFc2N * se < R ? kFc2N * se : R;
    const int nst = se - sb;
    for (int i = tid; i < re - rb; i += kThreads) rslot[i] = p.lslot[rb + i];
    __syncthreads();
    // down chunk of this thread
    const int ln = tid >> 5, lc = tid & 31;
    const int chunk = 32 * s + lc;
    const bool cin = chunk < p.cd;
    const uint32_t coff = p.dn_off + 16u * (uint32_t)chunk;
    const rsrc_t wr = buf_rsrc(p.bundles, p.all_bytes);
    // a chunk of this thread: half hl (waves 0-3 hi, 4-7 lo), token ta, rows 8ca ..
    const int hl = __builtin_amdgcn_readfirstlane(tid >> 8);   // wave-uniform
    const int ta = (tid >> 3) & 31, ca = tid & 7;
    const rsrc_t ar = buf_rsrc(p.la16 + (size_t)hl * p.Bm * p.LR, (uint32_t)p.B * p.LR * 2);
    const uint32_t ao = (uint32_t)(ta * p.LR + rb + 8 * ca) * 2;   // tokens past B read zeros
    // FUSED: partials of token ft, rows 4fc .. 4fc+3 of the step, slice k at
    // po + k * pstride (tokens past B read zeros)
    const int ft = tid >> 4, fc = tid & 15;
    const rsrc_t pr = buf_rsrc(p.part, FUSED ? (uint32_t)(p.ks * p.Bm * p.LR * 4) : 0u);
    const uint32_t pstride = (uint32_t)(p.Bm * p.LR * 4);
    const uint32_t po = (uint32_t)(ft * p.LR + rb + 4 * fc) * 4;
    u32x4 rv[kFc2Pre][4], ra[FUSED ? 1 : kFc2Pre], rp[FUSED ? kFc2Pre : 1][kFc2FuseKS];
    // the group's slots are staged in LDS, so a step's down loads do not wait
    // on a load of their slot
    auto load_step = [&](int st, int u) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rl = kFc2N * st + ln + 16 * j;
            const bool in = (st < nst) & (rb + rl < re);
            const int sl = rslot[in ? rl : 0];
            rv[u][j] = ld_stream(wr, (in & (sl >= 0) & cin) ? (uint32_t)sl * p.bundle_bytes + coff
                                                            : kOob);
        }
        if constexpr (FUSED) {
            const bool pin = (st < nst) & (ft < p.B);
#pragma unroll
            for (int k = 0; k < kFc2FuseKS; ++k)
                rp[u][k] = ld_shared(pr, (pin & (k < p.ks)) ? po + k * pstride + 4u * kFc2N * st
                                                            : kOob);
        } else {
            const bool ain = (st < nst) & (rb + kFc2N * st + 8 * ca < R);
            ra[u] = ld_shared(ar, ain ? ao + 2u * kFc2N * st : kOob);
        }
    };
    auto stage = [&](int st, int buf, int u) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = ln + 16 * j;
            *reinterpret_cast<u32x4 *>(&wl[buf][r * kWPitch + 8 * wl_chunk(r, lc)]) = rv[u][j];
        }
        if constexpr (FUSED) {
            // slice sums in slice order, ReLU, zero past the list, hi + lo
            f32x4v pv[kFc2FuseKS];
#pragma unroll
            for (int k = 0; k < kFc2FuseKS; ++k) pv[k] = __builtin_bit_cast(f32x4v, rp[u][k]);
            h4 hv, lv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float sum = 0.0f;
#pragma unroll
                for (int k = 0; k < kFc2FuseKS; ++k)
                    if (k < p.ks) sum += pv[k][e];
                const bool live = rb + kFc2N * st + 4 * fc + e < R;
                const float a = live ? fmaxf(sum, 0.0f) : 0.0f;
                hv[e] = (_Float16)a;
                lv[e] = (_Float16)(a - (float)hv[e]);
            }
            *reinterpret_cast<uint2 *>(&al[buf][ft * kAPitch + 4 * fc]) =
                __builtin_bit_cast(uint2, hv);
            *reinterpret_cast<uint2 *>(&al[buf][(kTile + ft) * kAPitch + 4 * fc]) =
                __builtin_bit_cast(uint2, lv);
        } else {
            // (a chunk across the list's end holds zeros past it: FC1 clears them)
            *reinterpret_cast<u32x4 *>(&al[buf][(hl * kTile + ta) * kAPitch + 8 * ca]) = ra[u];
        }
    };
    const int tk = lane & 31, hh = lane >> 5;
    const int jw = kTile * wave + tk;                     // output column within the slice
    f32x16 acc = zero16();
    if (nst > 0) {
#pragma unroll
        for (int u = 0; u < kFc2Pre; ++u) load_step(u, u);
        // steps past nst stage zeros: the loop body stays free of branches, so
        // the ring registers carry over without copies that would wait
        // step st from ring slot u (LDS buffer u % 2); NEXT: request step st + kFc2Pre
        auto step = [&](int st, int u, bool next) {
            const int buf = u & 1;
            stage(st, buf, u);
            if (next) load_step(st + kFc2Pre, u);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < kFc2N / 16; ++j) {
                const int k0 = 32 * hh + 8 * j;
                const h8 ahi = *reinterpret_cast<const h8 *>(&al[buf][tk * kAPitch + k0]);
                const h8 alo = *reinterpret_cast<const h8 *>(&al[buf][(kTile + tk) * kAPitch + k0]);
                h8 bv;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int r = k0 + e;
                    bv[e] = wl[buf][r * kWPitch + 8 * wl_chunk(r, jw >> 3) + (jw & 7)];
                }
                acc = mfma(ahi, bv, acc);
                acc = mfma(alo, bv, acc);
            }
        };
        // whole passes of kFc2Pre steps (the first peeled: the loop is entered
        // from a copy of its body, so the wait at its head need not cover every
        // load in flight), then the group's last 0-3 steps without requests
        int st0 = 0;
        if (nst >= kFc2Pre) {
#pragma unroll
            for (int u = 0; u < kFc2Pre; ++u) step(u, u, true);
            for (st0 = kFc2Pre; st0 + kFc2Pre <= nst; st0 += kFc2Pre) {
#pragma unroll
                for (int u = 0; u < kFc2Pre; ++u) step(st0 + u, u, true);
            }
        }
        static_assert(kFc2Pre == 4, "the tail below covers 0-3 steps");
        switch (nst - st0) {
        case 3: step(st0, 0, false); step(st0 + 1, 1, false); step(st0 + 2, 2, false); break;
        case 2: step(st0, 0, false); step(st0 + 1, 1, false); break;
        case 1: step(st0, 0, false); break;
        default: break;
        }
    }
    // group tile -> partial (k_fc2_fin adds the groups)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int t = acc_row(i, lane);
        const int m = kSliceOut * s + jw;
        if (t < p.B && m < p.d) p.partial[((size_t)g * p.B + t) * p.d + m] = acc[i];
    }
}

// Four outputs per thread: y[t][m..m+3] = the G group partials in group
// order, then b2, then the residual.
__global__ __launch_bounds__(256) void k_fc2_fin(const float *__restrict__ partial, int G, int B,
                                                 int d, const float *__restrict__ b2,
                                                 const float *__restrict__ resid,
                                                 float *__restrict__ y) {
    const int d4 = d / 4;
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= B * d4) return;
    const int t = idx / d4, m = 4 * (idx % d4);
    // all G loads in flight (unrolled to kGroups, clamped)
    float4 pv[kGroups];
#pragma unroll
    for (int gg = 0; gg < kGroups; ++gg)
        pv[gg] = *reinterpret_cast<const float4 *>(partial + ((size_t)(gg < G ? gg : 0) * B + t) * d + m);
    float4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int gg = 0; gg < kGroups; ++gg) {
        if (gg < G) {
            sum.x += pv[gg].x;
            sum.y += pv[gg].y;
            sum.z += pv[gg].z;
            sum.w += pv[gg].w;
        }
    }
    const float4 bb = *reinterpret_cast<const float4 *>(b2 + m);
    sum.x += bb.x;
    sum.y += bb.y;
    sum.z += bb.z;
    sum.w += bb.w;
    if (resid) {
        const float4 rr = *reinterpret_cast<const float4 *>(resid + (size_t)t * d + m);
        sum.x += rr.x;
        sum.y += rr.y;
        sum.z += rr.z;
        sum.w += rr.w;
    }
    *reinterpret_cast<float4 *>(y + (size_t)t * d + m) = sum;
}

inline hipEvent_t ev_start(const Trace *tr, int k) { return tr ? tr->ev[2 * k] : nullptr; }
inline hipEvent_t ev_stop(const Trace *tr, int k) { return tr ? tr->ev[2 * k + 1] : nullptr; }
#define ASF_LAUNCH(KID, F, GRID, BLK, ...) \
    hipExtLaunchKernelGGL(F, GRID, BLK, 0, s, ev_start(tr, KID), ev_stop(tr, KID), 0, __VA_ARGS__)

}  // namespace

int pred_slices(int d) { return (x16_pitch(d) + kPieceK - 1) / kPieceK; }

hipError_t launch_pred_mm(const LayerView &L, const float *x, int B, const Trace *tr,
                          hipStream_t s) {
    Fc1MmParams p = {};
    p.bundles = L.p1;
    p.bundle_bytes = (uint32_t)(L.cd * 16);          // P1 rows, d fp16 each
    p.cd = L.cd;
    p.b1 = L.c1;                                     // read, not added (k_pred_sum adds c1)
    p.add_b1 = 0;
    p.B = B;
    p.f = L.H;
    p.Bm = L.max_batch;
    p.LR = L.H;
    p.part = L.pred_part;
    p.ks = pred_slices(L.d);
    const int ncu = L.ncu > 0 ? L.ncu : 1;
    int GR = ncu / p.ks;
    const int gmin = (L.H + kFc1MaxRows - 1) / kFc1MaxRows;
    GR = GR > gmin ? GR : gmin;
    GR = GR < 1 ? 1 : GR;
    // the traced interval spans both kernels
    hipExtLaunchKernelGGL(k_pred_rows, dim3(GR * p.ks), dim3(kThreads), 0, s,
                          ev_start(tr, ASF_K_PRED_L1), nullptr, 0u, p, x, L.d);
    const int n = B * L.H > B * L.d / 8 ? B * L.H : B * L.d / 8;
    hipExtLaunchKernelGGL(k_pred_sum, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, s,
                          nullptr, ev_stop(tr, ASF_K_PRED_L1), 0u, (const float *)L.pred_part,
                          p.ks, L.max_batch, L.c1, x, B, L.d, L.H, L.h, L.h16, L.x16,
                          x16_pitch(L.d));
    return hipGetLastError();
}

hipError_t launch_score_mm(const LayerView &L, int B, const Trace *tr, hipStream_t s) {
    ASF_LAUNCH(ASF_K_SCORE, k_score_mm, dim3(L.nq), dim3(kThreads), (const u32x4 *)L.p2, L.c2,
               (const _Float16 *)L.h16, B, L.H, L.f, L.threshold, L.wbits, L.ubits);
    return hipGetLastError();
}

int fc1_slices(int d) { return (x16_pitch(d) + kSliceP * kPieceK - 1) / (kSliceP * kPieceK); }

// FC2 forms FC1's activations itself (no FC1 finishing kernel) for plain
// layers of at most kFc2FuseKS k slices, batches up to kFc2FuseB tokens and a
// neuron set (not every neuron): its workgroups then re-read few partials.
// Measured on the OPT-13B-shaped layer: B = 4 46.8 -> 45.3 us per step; at
// B = 16 / 32, and for all 20480 rows, the partial reads cost more than the
// finishing kernel saves.
constexpr int kFc2FuseB = 4;
bool fc2_fuses_fin(const LayerView &L, int B, bool all_rows) {
    return !all_rows && !L.gated && fc1_slices(L.d) <= kFc2FuseKS && B <= kFc2FuseB;
}

hipError_t launch_fc1_mm(const LayerView &L, const float *x, int B, int mode, const int32_t *ids,
                         const int32_t *n_ids, bool x16, const Trace *tr, hipStream_t s) {
    const int dp = x16_pitch(L.d);
    if (!x16) {
        // x as fp16 hi + lo first (the predictor writes this copy in a decode step)
        const int n8 = B * L.d / 8;
        hipLaunchKernelGGL(k_to_f16, dim3((n8 + 255) / 256 < 1024 ? (n8 + 255) / 256 : 1024),
                           dim3(256), 0, s, x, B, L.d, dp, L.max_batch, L.x16);
    }
    Fc1MmParams p;
    p.bundles = L.bundles;
    p.bundle_bytes = (uint32_t)(L.nmat * L.cd * 16);
    p.all_bytes = (uint32_t)((size_t)L.f * p.bundle_bytes);
    p.cd = L.cd;
    p.b1 = L.b1;
    p.x16 = L.x16;
    p.dp = dp;
    p.Bm = L.max_batch;
    p.B = B;
    p.f = L.f;
    p.nq = L.nq;
    p.mode = mode;
    p.ubits = L.ubits;
    p.ids = ids;
    p.n_ids = n_ids;
    p.inv = L.inv;
    p.lslot = L.lslot;
    p.la16 = L.la16;
    p.LR = L.nq * kRowsPerWG;
    p.rows = L.rows;
    p.part = L.fc1_part;
    p.ks = fc1_slices(L.d);
    p.add_b1 = 1;
    // KS slices x GR row groups: about one workgroup per CU (each holds
    // ~140 KiB of LDS), and enough groups that none takes more than
    // kFc1MaxRows rows
    const int gmin = (L.f + kFc1MaxRows - 1) / kFc1MaxRows;
    int GR = L.ncu / p.ks;
    GR = GR > gmin ? GR : gmin;
    // the traced interval spans both kernels (FC2 finishes FC1 itself when
    // fc2_fuses_fin: one kernel)
    const bool fused = fc2_fuses_fin(L, B, mode == 2);
    if (L.gated)
        hipExtLaunchKernelGGL(k_fc1_mm<true>, dim3(GR * p.ks), dim3(kThreads), 0, s,
                              ev_start(tr, ASF_K_FC1), nullptr, 0u, p);
    else
        hipExtLaunchKernelGGL(k_fc1_mm<false>, dim3(GR * p.ks), dim3(kThreads), 0, s,
                              ev_start(tr, ASF_K_FC1), fused ? ev_stop(tr, ASF_K_FC1) : nullptr,
                              0u, p);
    if (fused) return hipGetLastError();
    const int nfin = (B * (p.LR / 8) + 255) / 256;
    if (L.gated)
        hipExtLaunchKernelGGL(k_fc1_fin<true>, dim3(nfin), dim3(256), 0, s, nullptr,
                              ev_stop(tr, ASF_K_FC1), 0u, p);
    else
        hipExtLaunchKernelGGL(k_fc1_fin<false>, dim3(nfin), dim3(256), 0, s, nullptr,
                              ev_stop(tr, ASF_K_FC1), 0u, p);
    return hipGetLastError();
}

hipError_t launch_fc2_mm(const LayerView &L, int B, bool all_rows, const float *resid, float *y,
                         const Trace *tr, hipStream_t s) {
    Fc2MmParams p;
    p.bundles = L.bundles;
    p.bundle_bytes = (uint32_t)(L.nmat * L.cd * 16);
    p.all_bytes = (uint32_t)((size_t)L.f * p.bundle_bytes);
    p.dn_off = (uint32_t)((L.nmat - 1) * L.cd * 16);
    p.cd = L.cd;
    p.lslot = L.lslot;
    p.la16 = L.la16;
    p.LR = L.nq * kRowsPerWG;
    p.Bm = L.max_batch;
    p.rows = L.rows;
    p.d = L.d;
    p.B = B;
    p.partial = L.partial;
    p.part = L.fc1_part;
    p.ks = fc1_slices(L.d);
    // one workgroup per CU covers the grid: groups = 256 / slices, at most 16
    // (at least 8: d <= 8192 gives at most 32 slices)
    const int nslice = (L.cd + 31) / 32;
    int G = 256 / nslice;
    G = G < 1 ? 1 : (G > kGroups ? kGroups : G);
    p.groups = G;
    // the traced interval spans both kernels
    if (fc2_fuses_fin(L, B, all_rows))
        hipExtLaunchKernelGGL(k_fc2_mm<true>, dim3(nslice * G), dim3(kThreads), 0, s,
                              ev_start(tr, ASF_K_FC2), nullptr, 0u, p);
    else
        hipExtLaunchKernelGGL(k_fc2_mm<false>, dim3(nslice * G), dim3(kThreads), 0, s,
                              ev_start(tr, ASF_K_FC2), nullptr, 0u, p);
    const int n4 = B * (L.d / 4);
    hipExtLaunchKernelGGL(k_fc2_fin, dim3((n4 + 255) / 256), dim3(256), 0, s, nullptr,
                          ev_stop(tr, ASF_K_FC2), 0u, (const float *)L.partial, G, B, L.d, L.b2,
                          resid, y);
    return hipGetLastError();
}

}  // namespace asf
