// asf_batched.hip -- the batched form (B >= 2 tokens, fp16 weights) of the
// decode step on the matrix cores.  With B tokens sharing one step, every
// weight row the step touches meets all B tokens, so each phase is a skinny
// gathered GEMM: rows x tokens x k.  v_mfma_f32_32x32x16_f16 takes 32 rows x
// 32 tokens x 16 k per instruction (tokens past B are zero and load
// nothing).  Lane layout (gfx950): lane l supplies row (A) / column (B)
// l % 32 with the 8 consecutive k of group l / 32, and accumulator element
// i of lane l holds D[8(i/4) + 4(l/32) + i%4][l % 32].
//
//   predictor layer 1   rows of P1 x tokens, k = d, split over workgroups;
//                       a second kernel adds the partials (many workgroups:
//                       a last-arriver reduction costs an L2 write-back and
//                       an atomic round trip per workgroup, then a serial sum)
//   predictor layer 2   per owner: its 64 slot rows x tokens, k = H; then
//                       threshold and one ballot per token
//   FC1                 per owner: its union rows (compacted) x tokens
//   FC2                 tokens x outputs, k = the group's listed neurons;
//                       down segments go through LDS to be read transposed;
//                       a second kernel adds the groups' partials
//
// The predictor feeds x and h to the MFMA as fp16 hi + lo halves (two
// instructions per step), so its sums keep fp32 accuracy and the active
// sets stay those of an fp32 GEMV; FC1 and FC2 take x and a rounded to fp16
// once (their error stays orders of magnitude inside the output tolerance).
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

constexpr int kW = kThreads / 64;   // waves per workgroup
constexpr int kTile = 32;           // rows / tokens / outputs of one MFMA tile
constexpr int kSteps = 8;           // 16-k steps whose loads are in flight per wave
constexpr int kSliceOut = kTile * kW;  // FC2 outputs per workgroup (256)
constexpr int kMaxSplit = 8;        // predictor layer 1: k split over at most 8 workgroups

__device__ __forceinline__ f32x16 mfma(const h8 a, const h8 b, const f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.0f;
    return z;
}

__device__ __forceinline__ h8 zero_h8() {
    h8 z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (_Float16)0.0f;
    return z;
}

// row of accumulator element i in lane `lane` (its column is lane % 32)
__device__ __forceinline__ int acc_row(int i, int lane) {
    return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

// 8 consecutive fp32 values at p (16-byte aligned, always a valid address) as
// fp16; with HILO also the fp16 rounding of what the first rounding left
// out.  live == false gives zeros.
template <bool HILO>
__device__ __forceinline__ void frag_f32(const float *p, bool live, h8 &hi, h8 &lo) {
    const float4 *q = reinterpret_cast<const float4 *>(p);
    const float4 u = q[0], v = q[1];
    const float f[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float t = live ? f[j] : 0.0f;
        const _Float16 a = (_Float16)t;
        hi[j] = a;
        if constexpr (HILO) lo[j] = (_Float16)(t - (float)a);
    }
}

// Wave tiles -> LDS; returns nothing, caller synchronises.
__device__ __forceinline__ void tile_to_lds(float *dst, const f32x16 &acc, int lane) {
    const int col = lane & 31;
#pragma unroll
    for (int i = 0; i < 16; ++i) dst[acc_row(i, lane) * kTile + col] = acc[i];
}

// ---------------------------------------------------------------- predictor layer 1
// Workgroup (mt, ks): rows 32mt .. 32mt+31 of P1 over k in [ks*KW, (ks+1)*KW),
// KW = d / KS; wave w takes the w-th eighth of that range.  Wave tiles are
// added in wave order into the workgroup's partial tile; k_pred_fin adds the
// KS partial tiles of a row tile in ks order, then c1, then ReLU.
__global__ __launch_bounds__(kThreads) void k_pred_mm(const u32x4 *__restrict__ P1,
                                                      const float *__restrict__ x, int B, int d,
                                                      int H, int KS, float *__restrict__ part) {
    __shared__ float red[kW][kTile * kTile];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int mt = blockIdx.x / KS, ks = blockIdx.x % KS;
    const int KWw = d / KS / kW;                  // k per wave, a multiple of 16
    const int k_beg = ks * (d / KS) + wave * KWw, k_end = k_beg + KWw;
    const int g = lane >> 5, col = lane & 31;
    const int row = kTile * mt + col;
    const u32x4 *arow = P1 + (size_t)(row < H ? row : H - 1) * (d / 8);
    const bool tok = col < B;
    const float *xrow = x + (size_t)(tok ? col : 0) * d;
    f32x16 acc = zero16();
    for (int k0 = k_beg; k0 < k_end; k0 += 16 * kSteps) {
        u32x4 a[kSteps];
        h8 bh[kSteps], bl[kSteps];
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            const int kk = (k0 + 16 * s < k_end ? k0 + 16 * s : k_end - 16) + 8 * g;
            a[s] = arow[kk / 8];
            frag_f32<true>(xrow + kk, tok, bh[s], bl[s]);
        }
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            if (k0 + 16 * s < k_end) {
                const h8 av = __builtin_bit_cast(h8, a[s]);
                acc = mfma(av, bh[s], acc);
                acc = mfma(av, bl[s], acc);
            }
        }
    }
    tile_to_lds(red[wave], acc, lane);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int e = tid + kThreads * j;
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < kW; ++w) sum += red[w][e];
        part[((size_t)mt * KS + ks) * (kTile * kTile) + e] = sum;
    }
}

// Element e of row tile mt (row 32mt + e/32, token e%32): the KS partial
// tiles in ks order, then c1, then ReLU -> h and its fp16 hi/lo halves.  The
// grid also converts x to fp16 for the FC1 of the step.
__global__ __launch_bounds__(kThreads) void k_pred_fin(const float *__restrict__ part,
                                                       const float *__restrict__ c1,
                                                       const float *__restrict__ x, int B, int d,
                                                       int H, int KS, float *__restrict__ h,
                                                       _Float16 *__restrict__ h16,
                                                       _Float16 *__restrict__ x16) {
    const int gid = blockIdx.x * kThreads + threadIdx.x;
    const int mt = gid / (kTile * kTile), e = gid % (kTile * kTile);
    const int r = kTile * mt + e / kTile, t = e % kTile;
    if (r < H && t < B) {
        // all KS loads in flight (unrolled to the largest split, clamped)
        const float *pp = part + (size_t)mt * KS * (kTile * kTile) + e;
        float pv[kMaxSplit];
#pragma unroll
        for (int ks = 0; ks < kMaxSplit; ++ks) pv[ks] = pp[(size_t)(ks < KS ? ks : 0) * (kTile * kTile)];
        float sum = 0.0f;
#pragma unroll
        for (int ks = 0; ks < kMaxSplit; ++ks)
            if (ks < KS) sum += pv[ks];
        const float hv = fmaxf(sum + c1[r], 0.0f);
        const _Float16 hi = (_Float16)hv;
        h[(size_t)t * H + r] = hv;
        h16[(size_t)t * H + r] = hi;
        h16[(size_t)(B + t) * H + r] = (_Float16)(hv - (float)hi);
    }
    const int n8 = B * d / 8;
    for (int i = gid; i < n8; i += gridDim.x * kThreads) {
        h8 hv, unused;
        frag_f32<false>(x + (size_t)8 * i, true, hv, unused);
        *reinterpret_cast<h8 *>(x16 + (size_t)8 * i) = hv;
    }
}

// ---------------------------------------------------------------- operand tiles through LDS
// Both operands of a 32-row x 32-token x k product stream through LDS in
// chunks of CW 16-byte chunks (8*CW k) per row: the weight tile (32 rows)
// and the token tile (32 token rows of fp16).  Thread t loads chunk t%16
// (and t%16 + 16) of row t/16, so a wave instruction covers 4 rows x 256
// contiguous bytes.  Loads run kPre chunks ahead into registers, always
// from clamped addresses and zeroed afterwards (a load under a lane
// condition makes the compiler wait for every outstanding load before the
// next LDS store, which would cancel the prefetch).  A chunk is stored to one
// of two LDS buffers with the 16-byte chunk index XOR-ed with row % 16, so a
// fragment read (32 rows at one chunk) hits distinct banks.  Wave w
// multiplies its CW/16 of the CW/2 MFMA steps of every chunk: a k split over
// the waves, whose 8 partial tiles are added in wave order at the end.
constexpr int kPre = 4;                      // chunks in flight per thread

template <int CW> struct Geo {
    static constexpr int LPT = CW / 16;      // loads per thread per tile chunk
    static constexpr int SPW = CW / 16;      // MFMA steps per wave per chunk
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

// ---------------------------------------------------------------- FC1
struct Fc1MmParams {
    const u32x4 *bundles;
    size_t bstride;      // chunks per bundle
    int cd;              // chunks per d row
    const float *b1;
    const _Float16 *x16; // x as fp16 [B][d]
    int B, d, f, nq;
    int mode;            // 0 union of the last prediction, 1 caller ids, 2 all
    const uint64_t *ubits;
    const int32_t *ids;
    const int32_t *n_ids;
    const int32_t *inv;
    int32_t *lslot;      // [rows] slot of list row r (-1: a skipped caller id)
    float *la;           // [rows][max_batch]
    int max_batch;
    int32_t *rows;       // number of list rows
    int ncu;             // compute units
    int per_cu;          // workgroups resident per CU at once (LDS, registers)
};

// x -> fp16 [B][d] (for FC1 calls that follow no predictor pass)
__global__ void k_to_f16(const float *__restrict__ x, int n, _Float16 *__restrict__ x16) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
        x16[i] = (_Float16)x[i];
}

// The FC1 list: mode 0 the union of the last prediction, owner by owner
// (row r is the (r - pre[q])-th set bit i of owner q, slot q + nq*i, for the
// owner with pre[q] <= r < pre[q+1], pre the popcount prefix); mode 1 the
// caller's ids in list order; mode 2 every slot.  Workgroup b takes rows
// Rb .. Rb+R-1 as one tile streamed with the token tile of x (fp16) over k = d
// in chunks of 256 k.  While the list needs at most one 32-row workgroup
// per CU it is spread over one workgroup per CU (R = its length over the
// CUs, at least kFc1MinRows); a longer list is spread evenly over the
// workgroups resident at once
// (R = its length over them, at least kFc1MinRows; the tile's other rows are
// dead), since a CU holding two workgroups runs each ~30% slower and an
// uneven split leaves the kernel waiting on the doubled CUs.  a = ReLU(up . x + b1) (gated: ReLU(gate . x +
// b1) * (up . x)), written to la[r][t] and lslot[r].
constexpr int kFc1MinRows = 16;

template <bool GATED>
__global__ __launch_bounds__(kThreads) void k_fc1_mm(Fc1MmParams p) {
    constexpr int CW = 32;
    constexpr int EL = Geo<CW>::ELEMS;
    constexpr int NT = GATED ? 3 : 2;                // staged tiles: [gate,] up, x
    constexpr int PRE = kPre;                        // chunks in flight per thread
    __shared__ u32x4 smem[2 * NT * EL];              // chunks; before: owner words; after: wave tiles
    __shared__ float gsum[GATED ? kTile * kTile : 1];
    __shared__ int pre[kMaxFfn / 64 + 1];
    __shared__ int wave_tot[kW];
    __shared__ int rslot[kTile];
    __shared__ int nrows_lds;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // rows per workgroup from the list length (the same in every workgroup)
    auto tile_rows = [&](int n) {
        if (n <= kTile * p.ncu) {
            // one workgroup per CU at most: spread the list over every CU
            const int r = (n + p.ncu - 1) / p.ncu;
            return r < kFc1MinRows ? kFc1MinRows : r;
        }
        const int nw = p.per_cu * p.ncu;
        const int r = (n + nw - 1) / nw;
        return r < kFc1MinRows ? kFc1MinRows : (r > kTile ? kTile : r);
    };
    int R = kTile, r0 = 0;
    // ---- the list's length and this tile's slots
    if (p.mode == 0) {
        uint64_t *vb = reinterpret_cast<uint64_t *>(smem);
        const int nq = p.nq;
        for (int q = tid; q < nq; q += kThreads) vb[q] = p.ubits[q];
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
        __syncthreads();
        R = tile_rows(nrows_lds);
        r0 = R * blockIdx.x;
        if (tid < kTile) {
            const int r = r0 + tid;
            int slot = -1;
            if (tid < R && r < nrows_lds) {
                int lo = 0, hi = nq;                 // largest q with pre[q] <= r
                while (hi - lo > 1) {
                    const int mid = (lo + hi) >> 1;
                    if (pre[mid] <= r) lo = mid;
                    else hi = mid;
                }
                slot = lo + nq * nth_set_bit(vb[lo], r - pre[lo]);
            }
            rslot[tid] = slot;
        }
    } else {
        if (tid == 0) {
            int n = p.f;
            if (p.mode == 1) {
                n = *p.n_ids;
                n = n < 0 ? 0 : (n > p.f ? p.f : n);
            }
            nrows_lds = n;
        }
        __syncthreads();
        R = tile_rows(nrows_lds);
        r0 = R * blockIdx.x;
        if (tid < kTile) {
            const int r = r0 + tid;
            int slot = -1;
            if (tid < R && r < nrows_lds) {
                if (p.mode == 2) {
                    slot = r;
                } else {
                    const int id = p.ids[r];
                    slot = (unsigned)id < (unsigned)p.f ? p.inv[id] : -1;
                    if ((unsigned)slot >= (unsigned)p.f) slot = -1;
                }
            }
            rslot[tid] = slot;
        }
    }
    __syncthreads();
    const int nrows = nrows_lds;
    // (the list length is stored after the tile: a global store in flight
    // would make the compiler wait for every load of the ring)
    if (r0 >= nrows) {
        if (blockIdx.x == 0 && tid == 0) *p.rows = nrows;
        return;
    }
    // ---- the tile over k = d
    const int C = p.cd;
    const int nch = (C + CW - 1) / CW;
    const int lrow = tid / 16, lc = tid % 16;
    const int myslot = rslot[lrow];
    const bool live = myslot >= 0;
    constexpr int UP = GATED ? 1 : 0;
    const u32x4 *bp = p.bundles + (size_t)(live ? myslot : 0) * p.bstride;
    const u32x4 *rpu = bp + (size_t)UP * C, *rpg = bp;
    const bool tokr = lrow < p.B;
    const u32x4 *xr = reinterpret_cast<const u32x4 *>(p.x16 + (size_t)(tokr ? lrow : 0) * p.d);
    // chunks past nch load zeros (chunk indices past C are clamped and
    // zeroed), so the loop body stays free of branches and the ring registers
    // carry over without copies that would wait
    u32x4 ra[PRE][NT][Geo<CW>::LPT];
    auto load = [&](int ch, u32x4 (&v)[NT][Geo<CW>::LPT]) {
        ld_chunk<CW>(rpu, C, ch, lc, v[0]);
        ld_chunk<CW>(xr, C, ch, lc, v[1]);
        if constexpr (GATED) ld_chunk<CW>(rpg, C, ch, lc, v[NT - 1]);
    };
#pragma unroll
    for (int u = 0; u < PRE; ++u) load(u, ra[u]);
    f32x16 accu = zero16(), accg = zero16();
    auto pass = [&](int ch0) {
#pragma unroll
        for (int u = 0; u < PRE; ++u) {
            const int ch = ch0 + u;
            u32x4 *bufp = smem + (u & 1) * NT * EL;
            st_chunk<CW>(bufp, lrow, lc, live, C, ch, ra[u][0]);
            st_chunk<CW>(bufp + EL, lrow, lc, tokr, C, ch, ra[u][1]);
            if constexpr (GATED) st_chunk<CW>(bufp + (NT - 1) * EL, lrow, lc, live, C, ch, ra[u][NT - 1]);
            load(ch + PRE, ra[u]);
            __syncthreads();
#pragma unroll
            for (int k = 0; k < Geo<CW>::SPW; ++k) {
                const int st = Geo<CW>::SPW * wave + k;
                const h8 bx = frag<CW>(bufp + EL, st, lane);
                accu = mfma(frag<CW>(bufp, st, lane), bx, accu);
                if constexpr (GATED) accg = mfma(frag<CW>(bufp + (NT - 1) * EL, st, lane), bx, accg);
            }
        }
    };
    // the first pass is peeled (nch >= 1): the loop is then entered from a
    // copy of its own body, with the ring's loads in the loop's order, so the
    // wait at the loop head can stay fine-grained (entered from the prologue
    // it would have to wait for every load in flight, on every pass)
    pass(0);
    for (int ch0 = PRE; ch0 < nch; ch0 += PRE) pass(ch0);
    // ---- epilogue
    float *red = reinterpret_cast<float *>(smem);
    float v[2];
    if constexpr (GATED) {
        __syncthreads();
        tile_to_lds(red + wave * kTile * kTile, accg, lane);
        __syncthreads();
        tile_sum(red, v);
#pragma unroll
        for (int j = 0; j < 2; ++j) gsum[tid + kThreads * j] = v[j];
    }
    __syncthreads();
    tile_to_lds(red + wave * kTile * kTile, accu, lane);
    __syncthreads();
    tile_sum(red, v);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int e = tid + kThreads * j;
        const int rr = e / kTile, t = e % kTile, r = r0 + rr;
        if (rr >= R || r >= nrows || t >= p.B) continue;
        const int sl = rslot[rr];
        float a = 0.0f;
        if (sl >= 0) {
            if constexpr (GATED) a = fmaxf(gsum[e] + p.b1[sl], 0.0f) * v[j];
            else a = fmaxf(v[j] + p.b1[sl], 0.0f);
        }
        p.la[(size_t)r * p.max_batch + t] = a;
        if (t == 0) p.lslot[r] = sl;
    }
    if (blockIdx.x == 0 && tid == 0) *p.rows = nrows;
}

// ---------------------------------------------------------------- FC2
struct Fc2MmParams {
    const u32x4 *bundles;
    size_t bstride;      // chunks per bundle
    int dn_off;          // chunk offset of the down column in a bundle
    int cd;              // chunks per down column
    const int32_t *lslot;
    const float *la;
    const int32_t *rows;
    int max_batch;
    int d, B;
    const float *b2;
    const float *resid;
    float *y;
    float *partial;      // [groups][B][d]
    int groups;          // list-row ranges (<= kGroups)
};

constexpr int kFc2N = 64;                   // neurons per step (4 MFMA k-steps)
constexpr int kWPitch = kSliceOut + 8;      // halfs per staged down row
constexpr int kAPitch = kFc2N + 8;          // halfs per staged token row of a
constexpr int kFc2Pre = 4;                  // steps in flight per thread
constexpr int kFc2Rows = 8192;              // list rows per group (f <= 65536, >= 8 groups)

// Workgroup (slice s, group g): outputs 256s .. 256s+255 over list rows
// [g*R/G, (g+1)*R/G).  Per step of 64 rows each thread loads four 16-byte
// chunks of down segments (row tid/32 + 16j, chunk tid%32) and four a values
// (row tid/32 + 16j, token tid%32), kFc2Pre steps ahead; the step is staged
// in LDS (double buffered) and wave w multiplies tokens x its 32 outputs x
// 64 rows, reading each lane's 8 rows of one output column transposed.
// Group tiles go to `partial`; k_fc2_fin adds the G in group order, then b2,
// then the residual.
__global__ __launch_bounds__(kThreads) void k_fc2_mm(Fc2MmParams p) {
    __shared__ __attribute__((aligned(16))) _Float16 wl[2][kFc2N * kWPitch];
    __shared__ __attribute__((aligned(16))) _Float16 al[2][kTile * kAPitch];
    __shared__ int rslot[kFc2Rows];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = p.groups;
    const int nslice = gridDim.x / G;
    const int s = blockIdx.x % nslice, g = blockIdx.x / nslice;
    const int R = *p.rows;
    const int rb = (int)((long long)R * g / G), re = (int)((long long)R * (g + 1) / G);
    const int nst = (re - rb + kFc2N - 1) / kFc2N;
    for (int i = tid; i < re - rb; i += kThreads) rslot[i] = p.lslot[rb + i];
    __syncthreads();
    const int ln = tid / kTile, lc = tid % kTile;
    const int chunk = s * (kSliceOut / 8) + lc;
    const bool cin = chunk < p.cd;
    const u32x4 *dbase = p.bundles + p.dn_off + (cin ? chunk : 0);
    const bool tok_a = lc < p.B;
    u32x4 rv[kFc2Pre][4];
    float ra[kFc2Pre][4];
    // the group's list slots are staged in LDS, so a step's down-segment
    // loads do not wait on a load of their slot
    // loads from clamped addresses; the values are zeroed only when staged,
    // a ring period later, so that no instruction touches them before then
    auto row_ok = [&](int st, int j) {                   // branch free (bitwise and)
        const int rl = st * kFc2N + ln + 16 * j;              // row within the group
        const bool in = (st < nst) & (rb + rl < re);
        return in & (rslot[in ? rl : 0] >= 0);
    };
    auto load_step = [&](int st, u32x4 (&v)[4], float (&a)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rl = st * kFc2N + ln + 16 * j;
            const bool in = (st < nst) & (rb + rl < re);
            const int sl = rslot[in ? rl : 0];
            v[j] = dbase[(size_t)(sl >= 0 ? sl : 0) * p.bstride];
            a[j] = p.la[(size_t)(in ? rb + rl : rb) * p.max_batch + (tok_a ? lc : 0)];
        }
    };
    auto stage = [&](int st, int buf, const u32x4 (&v)[4], const float (&a)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool ok = row_ok(st, j);
            *reinterpret_cast<u32x4 *>(&wl[buf][(ln + 16 * j) * kWPitch + 8 * lc]) = sel4(ok & cin, v[j]);
            al[buf][lc * kAPitch + ln + 16 * j] = (_Float16)((ok & tok_a) ? a[j] : 0.0f);
        }
    };
    const int gk = lane >> 5, col = lane & 31;
    const int jw = kTile * wave + col;
    f32x16 acc = zero16();
    if (nst > 0) {
#pragma unroll
        for (int u = 0; u < kFc2Pre; ++u) load_step(u, rv[u], ra[u]);
        // steps past nst stage zeros: the loop body stays free of branches, so
        // the ring registers carry over without copies that would wait
        auto pass = [&](int st0) {
#pragma unroll
            for (int u = 0; u < kFc2Pre; ++u) {
                const int st = st0 + u;
                const int buf = u & 1;
                stage(st, buf, rv[u], ra[u]);
                load_step(st + kFc2Pre, rv[u], ra[u]);
                __syncthreads();
#pragma unroll
                for (int k = 0; k < kFc2N / 16; ++k) {
                    const h8 av = *reinterpret_cast<const h8 *>(&al[buf][col * kAPitch + 16 * k + 8 * gk]);
                    h8 bv;
#pragma unroll
                    for (int j = 0; j < 8; ++j) bv[j] = wl[buf][(16 * k + 8 * gk + j) * kWPitch + jw];
                    acc = mfma(av, bv, acc);
                }
            }
        };
        // first pass peeled: the loop is entered from a copy of its body, so
        // the wait at its head need not cover every load in flight
        pass(0);
        for (int st0 = kFc2Pre; st0 < nst; st0 += kFc2Pre) pass(st0);
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

// split of the predictor's k over workgroups: the largest power of two <=
// kMaxSplit with d a multiple of 128 * KS (every wave then takes a multiple
// of 16 k)
int pred_mm_splits(int d) {
    int ks = kMaxSplit;
    while (ks > 1 && d % (128 * ks) != 0) ks >>= 1;
    return ks;
}

hipError_t launch_pred_mm(const LayerView &L, const float *x, int B, const Trace *tr,
                          hipStream_t s) {
    const int mt = (L.H + kTile - 1) / kTile, ks = pred_mm_splits(L.d);
    // the traced interval spans both kernels
    hipExtLaunchKernelGGL(k_pred_mm, dim3(mt * ks), dim3(kThreads), 0, s,
                          ev_start(tr, ASF_K_PRED_L1), nullptr, 0u, (const u32x4 *)L.p1, x, B,
                          L.d, L.H, ks, L.pred_part);
    const int nfin = mt * (kTile * kTile) / kThreads;
    hipExtLaunchKernelGGL(k_pred_fin, dim3(nfin), dim3(kThreads), 0, s, nullptr,
                          ev_stop(tr, ASF_K_PRED_L1), 0u, (const float *)L.pred_part, L.c1, x, B,
                          L.d, L.H, ks, L.h, L.h16, L.x16);
    return hipGetLastError();
}

hipError_t launch_score_mm(const LayerView &L, int B, const Trace *tr, hipStream_t s) {
    ASF_LAUNCH(ASF_K_SCORE, k_score_mm, dim3(L.nq), dim3(kThreads), (const u32x4 *)L.p2, L.c2,
               (const _Float16 *)L.h16, B, L.H, L.f, L.threshold, L.wbits, L.ubits);
    return hipGetLastError();
}

hipError_t launch_fc1_mm(const LayerView &L, const float *x, int B, int mode, const int32_t *ids,
                         const int32_t *n_ids, bool x16, const Trace *tr, hipStream_t s) {
    if (!x16) {
        // x as fp16 first (the predictor writes this copy in a decode step)
        const int n = B * L.d;
        hipLaunchKernelGGL(k_to_f16, dim3((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024),
                           dim3(256), 0, s, x, n, L.x16);
    }
    Fc1MmParams p;
    p.bundles = (const u32x4 *)L.bundles;
    p.bstride = (size_t)L.nmat * L.cd;
    p.cd = L.cd;
    p.b1 = L.b1;
    p.x16 = L.x16;
    p.B = B;
    p.d = L.d;
    p.f = L.f;
    p.nq = L.nq;
    p.mode = mode;
    p.ubits = L.ubits;
    p.ids = ids;
    p.n_ids = n_ids;
    p.inv = L.inv;
    p.lslot = L.lslot;
    p.la = L.la;
    p.max_batch = L.max_batch;
    p.rows = L.rows;
    p.ncu = L.ncu;
    p.per_cu = L.gated ? 1 : 2;
    // enough workgroups for any list length (at most f rows): 32 rows each,
    // or the spread (at most per_cu per CU); the rest return at once
    const int g32 = (L.f + kTile - 1) / kTile;
    const dim3 grid(g32 > p.per_cu * p.ncu ? g32 : p.per_cu * p.ncu);
    if (L.gated) ASF_LAUNCH(ASF_K_FC1, k_fc1_mm<true>, grid, dim3(kThreads), p);
    else ASF_LAUNCH(ASF_K_FC1, k_fc1_mm<false>, grid, dim3(kThreads), p);
    return hipGetLastError();
}

hipError_t launch_fc2_mm(const LayerView &L, int B, bool listed, const float *resid, float *y,
                         const Trace *tr, hipStream_t s) {
    (void)listed;   // the batched list always carries its slots
    Fc2MmParams p;
    p.bundles = (const u32x4 *)L.bundles;
    p.bstride = (size_t)L.nmat * L.cd;
    p.dn_off = (L.nmat - 1) * L.cd;
    p.cd = L.cd;
    p.lslot = L.lslot;
    p.la = L.la;
    p.rows = L.rows;
    p.max_batch = L.max_batch;
    p.d = L.d;
    p.B = B;
    p.b2 = L.b2;
    p.resid = resid;
    p.y = y;
    p.partial = L.partial;
    // one workgroup per CU covers the grid: groups = 256 / slices, at most 16
    const int nslice = (L.d + kSliceOut - 1) / kSliceOut;
    int G = 256 / nslice;
    G = G < 1 ? 1 : (G > kGroups ? kGroups : G);
    p.groups = G;
    // the traced interval spans both kernels
    hipExtLaunchKernelGGL(k_fc2_mm, dim3(nslice * G), dim3(kThreads), 0, s,
                          ev_start(tr, ASF_K_FC2), nullptr, 0u, p);
    const int n4 = B * (L.d / 4);
    hipExtLaunchKernelGGL(k_fc2_fin, dim3((n4 + 255) / 256), dim3(256), 0, s, nullptr,
                          ev_stop(tr, ASF_K_FC2), 0u, (const float *)L.partial, G, B, L.d, L.b2,
                          resid, y);
    return hipGetLastError();
}

}  // namespace asf
