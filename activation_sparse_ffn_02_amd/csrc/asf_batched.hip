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
//                       the last workgroup of a row tile adds the partials
//   predictor layer 2   per owner: its 64 slot rows x tokens, k = H; then
//                       threshold and one ballot per token
//   FC1                 per owner: its union rows (compacted) x tokens
//   FC2                 tokens x outputs, k = the group's listed neurons;
//                       down segments go through LDS to be read transposed
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

// Agent-scope arrival of this workgroup at counter c (after every thread's
// global stores); true for the last of `n` arrivals, which also resets it.
__device__ __forceinline__ bool arrive_last(unsigned *c, unsigned n, int *flag_lds) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const unsigned old = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = old == n - 1;
        if (last) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        *flag_lds = last;
    }
    __syncthreads();
    return *flag_lds != 0;
}

// ---------------------------------------------------------------- predictor layer 1
// Workgroup (mt, ks): rows 32mt .. 32mt+31 of P1 over k in [ks*KW, (ks+1)*KW),
// KW = d / KS; wave w takes the w-th eighth of that range.  Wave tiles are
// added in wave order; with KS > 1 the KS workgroup tiles of a row tile meet
// in `part` and the last to arrive adds them in ks order, then c1, then ReLU.
__global__ __launch_bounds__(kThreads) void k_pred_mm(const u32x4 *__restrict__ P1,
                                                      const float *__restrict__ c1,
                                                      const float *__restrict__ x, int B, int d,
                                                      int H, int KS, float *__restrict__ part,
                                                      unsigned *__restrict__ arrive,
                                                      float *__restrict__ h) {
    __shared__ float red[kW][kTile * kTile];
    __shared__ int last_lds;
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
    float v[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int e = tid + kThreads * j;
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < kW; ++w) sum += red[w][e];
        v[j] = sum;
    }
    if (KS > 1) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
            part[((size_t)mt * KS + ks) * (kTile * kTile) + tid + kThreads * j] = v[j];
        if (!arrive_last(arrive + mt, (unsigned)KS, &last_lds)) return;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            float sum = 0.0f;
            for (int kk = 0; kk < KS; ++kk)
                sum += part[((size_t)mt * KS + kk) * (kTile * kTile) + tid + kThreads * j];
            v[j] = sum;
        }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int e = tid + kThreads * j;
        const int r = kTile * mt + e / kTile, t = e % kTile;
        if (r < H && t < B) h[(size_t)t * H + r] = fmaxf(v[j] + c1[r], 0.0f);
    }
}

// ---------------------------------------------------------------- predictor layer 2
// Owner q: rows i = 0..63 (slot q + nq*i) in two 32-row tiles; wave w takes
// tile w & 1 and the (w >> 1)-th quarter of the 16-k steps over H.  The
// quarter tiles are added in order, then c2; wave w ballots tokens w, w+8,
// ... into the per-token owner words; the union is their OR.
__global__ __launch_bounds__(kThreads) void k_score_mm(const u32x4 *__restrict__ P2,
                                                       const float *__restrict__ c2,
                                                       const float *__restrict__ h, int B, int H,
                                                       int f, float theta,
                                                       uint64_t *__restrict__ wbits,
                                                       uint64_t *__restrict__ ubits) {
    __shared__ float red[kW][kTile * kTile];
    __shared__ uint64_t uw[kW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q = blockIdx.x, nq = gridDim.x;
    const int tile = wave & 1, quarter = wave >> 1;
    const int g = lane >> 5, col = lane & 31;
    const int C = H / 8;                              // 8-k chunks per row
    const int nst = (C + 1) / 2;                      // 16-k steps (the last may be half)
    const int st_beg = quarter * nst / 4, st_end = (quarter + 1) * nst / 4;
    int slot = q + nq * (kTile * tile + col);
    slot = slot < f ? slot : f - 1;
    const u32x4 *arow = P2 + (size_t)slot * C;
    const bool tok = col < B;
    const float *hrow = h + (size_t)(tok ? col : 0) * H;
    f32x16 acc = zero16();
    for (int s0 = st_beg; s0 < st_end; s0 += kSteps) {
        u32x4 a[kSteps];
        h8 bh[kSteps], bl[kSteps];
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            const int st = s0 + s < st_end ? s0 + s : st_end - 1;
            const int c = 2 * st + g;
            const bool in = c < C;
            const int cc = in ? c : C - 1;
            a[s] = in ? arow[cc] : u32x4{0u, 0u, 0u, 0u};
            frag_f32<true>(hrow + 8 * cc, tok && in, bh[s], bl[s]);
        }
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            if (s0 + s < st_end) {
                const h8 av = __builtin_bit_cast(h8, a[s]);
                acc = mfma(av, bh[s], acc);
                acc = mfma(av, bl[s], acc);
            }
        }
    }
    tile_to_lds(red[wave], acc, lane);
    __syncthreads();
    // score of row i (0..63), token t: tiles i / 32, quarters in order
    const int i = lane;
    const int slot_i = q + nq * i;
    const bool valid_i = slot_i < f;
    const float bias = c2[valid_i ? slot_i : f - 1];
    uint64_t u = 0;
    for (int t = wave; t < B; t += kW) {
        const int e = (i % kTile) * kTile + t, tl = i / kTile;
        float sc = 0.0f;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) sc += red[tl + 2 * qq][e];
        const uint64_t m = __ballot(valid_i && sc + bias > theta);
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
    const float *x;
    int B, d, f;
    int mode;            // 0 union of the last prediction, 1 caller ids, 2 all
    const uint64_t *ubits;
    const int32_t *ids;
    const int32_t *n_ids;
    const int32_t *inv;
    uint64_t *vbits;
    int32_t *lslot;
    float *la;
    int max_batch;
};

// Owner q: its listed neurons (rank r = r-th set bit) are rows of up to two
// 32-row tiles; with one tile all 8 waves split k, with two each tile gets 4
// waves.  Wave sums are added in k order; a = ReLU(up . x + b1) or, gated,
// ReLU(gate . x + b1) * (up . x); written to la[q][r][t] and lslot[q][r].
template <bool GATED>
__global__ __launch_bounds__(kThreads) void k_fc1_mm(Fc1MmParams p) {
    __shared__ int slot_lds[kRowsPerWG];
    __shared__ int crow[kRowsPerWG];
    __shared__ uint64_t valid_lds;
    __shared__ float red[GATED ? 2 : 1][kW][kTile * kTile];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q = blockIdx.x, nq = gridDim.x;
    if (tid < kRowsPerWG) {
        const int i = tid;
        int slot = -1;
        if (p.mode == 1) {
            int n = *p.n_ids;
            n = n < 0 ? 0 : (n > p.f ? p.f : n);
            const int e = q + nq * i;
            if (e < n) {
                const int id = p.ids[e];
                slot = (unsigned)id < (unsigned)p.f ? p.inv[id] : -1;
                if ((unsigned)slot >= (unsigned)p.f) slot = -1;
            }
        } else {
            const int s = q + nq * i;
            if (s < p.f && (p.mode == 2 || ((p.ubits[q] >> i) & 1ull))) slot = s;
        }
        slot_lds[i] = slot;
        const uint64_t b = __ballot(slot >= 0);
        if (slot >= 0) crow[__popcll(b & ((1ull << i) - 1ull))] = slot;
        if (i == 0) valid_lds = b;
    }
    __syncthreads();
    const uint64_t valid = valid_lds;
    if (tid == 0) p.vbits[q] = valid;
    const int n = __popcll(valid);
    if (n == 0) return;
    const int ntiles = (n + kTile - 1) / kTile;
    const int tile = wave % ntiles, nk = kW / ntiles, kp = wave / ntiles;
    const int g = lane >> 5, col = lane & 31;
    const int r = kTile * tile + col;
    const bool live = r < n;
    const int slot = crow[live ? r : 0];
    constexpr int UP = GATED ? 1 : 0;
    const u32x4 *bp = p.bundles + (size_t)slot * p.bstride;
    const bool tok = col < p.B;
    const float *xrow = p.x + (size_t)(tok ? col : 0) * p.d;
    const int nst = p.cd / 2;                         // 16-k steps (cd is even)
    const int st_beg = kp * nst / nk, st_end = (kp + 1) * nst / nk;
    f32x16 acc = zero16(), accg = zero16();
    for (int s0 = st_beg; s0 < st_end; s0 += kSteps) {
        u32x4 a[kSteps], ag[kSteps];
        h8 bx[kSteps], unused[kSteps];
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            const int st = s0 + s < st_end ? s0 + s : st_end - 1;
            const int c = 2 * st + g;
            a[s] = live ? bp[(size_t)UP * p.cd + c] : u32x4{0u, 0u, 0u, 0u};
            if constexpr (GATED) ag[s] = live ? bp[c] : u32x4{0u, 0u, 0u, 0u};
            frag_f32<false>(xrow + 8 * c, tok, bx[s], unused[s]);
        }
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            if (s0 + s < st_end) {
                acc = mfma(__builtin_bit_cast(h8, a[s]), bx[s], acc);
                if constexpr (GATED) accg = mfma(__builtin_bit_cast(h8, ag[s]), bx[s], accg);
            }
        }
    }
    tile_to_lds(red[0][wave], acc, lane);
    if constexpr (GATED) tile_to_lds(red[GATED ? 1 : 0][wave], accg, lane);
    __syncthreads();
    for (int e2 = tid; e2 < ntiles * kTile * kTile; e2 += kThreads) {
        const int tl = e2 / (kTile * kTile), e = e2 % (kTile * kTile);
        const int rr = kTile * tl + e / kTile, t = e % kTile;
        if (rr >= n || t >= p.B) continue;
        float su = 0.0f, sg = 0.0f;
        for (int k = 0; k < nk; ++k) {
            su += red[0][tl + ntiles * k][e];
            if constexpr (GATED) sg += red[GATED ? 1 : 0][tl + ntiles * k][e];
        }
        const int sl = crow[rr];
        const float a = GATED ? fmaxf(sg + p.b1[sl], 0.0f) * su : fmaxf(su + p.b1[sl], 0.0f);
        const size_t ent = (size_t)q * kRowsPerWG + rr;
        p.la[ent * p.max_batch + t] = a;
        if (t == 0) p.lslot[ent] = sl;
    }
}

// ---------------------------------------------------------------- FC2
struct Fc2MmParams {
    const u32x4 *bundles;
    size_t bstride;      // chunks per bundle
    int dn_off;          // chunk offset of the down column in a bundle
    int cd;              // chunks per down column
    const uint64_t *vbits;
    const int32_t *lslot;
    int listed;
    const float *la;
    int max_batch;
    int nq, d, B;
    const float *b2;
    const float *resid;
    float *y;
    float *partial;      // [kGroups][B][d]
    unsigned *arrive;    // per slice
};

constexpr int kMaxProd = kMaxFfn / kRowsPerWG / kGroups + 1;
constexpr int kFc2K = 16;                   // neurons per MFMA step
constexpr int kWPitch = kSliceOut + 8;      // halfs per staged down row (16-byte multiple)
constexpr int kAPitch = kFc2K + 8;          // halfs per staged token row of a

// Workgroup (slice s, group g): outputs 256s .. 256s+255, neurons listed by
// owners g, g+16, ...  Per step of 16 neurons each thread loads one 16-byte
// chunk of one down segment (neuron tid / 32, chunk tid % 32) and one a
// value (neuron tid / 32, token tid % 32), kSteps steps ahead; the step is
// written to LDS (double buffered) and wave w multiplies tokens x its 32
// outputs x 16 neurons, reading each lane's 8 neurons of one output column
// transposed from LDS.  Group tiles meet in `partial`; the last group to
// arrive at the slice adds the 16 in group order, then b2, then the residual.
__global__ __launch_bounds__(kThreads) void k_fc2_mm(Fc2MmParams p) {
    __shared__ uint64_t vb[kMaxProd];
    __shared__ int pre[kMaxProd + 1];
    __shared__ int2 tab[kMaxProd * kRowsPerWG];
    __shared__ __attribute__((aligned(16))) _Float16 wl[2][kFc2K * kWPitch];
    __shared__ __attribute__((aligned(16))) _Float16 al[2][kTile * kAPitch];
    __shared__ int last_lds;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nslice = gridDim.x / kGroups;
    const int s = blockIdx.x % nslice, g = blockIdx.x / nslice;
    const int np = g < p.nq ? (p.nq - g + kGroups - 1) / kGroups : 0;
    if (tid < np) vb[tid] = p.vbits[g + kGroups * tid];
    __syncthreads();
    if (tid < 64) {
        const int c = tid < np ? __popcll(vb[tid]) : 0;
        int incl = c;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(incl, o, 64);
            if (tid >= o) incl += v;
        }
        if (tid < np) pre[tid] = incl - c;
        if (tid == 63) pre[np] = incl;
    }
    __syncthreads();
    const int ng = pre[np];
    for (int idx = tid; idx < np * kRowsPerWG; idx += kThreads) {
        const int k = idx / kRowsPerWG, i = idx % kRowsPerWG;
        const uint64_t m = vb[k];
        if ((m >> i) & 1ull) {
            const int r = __popcll(m & ((1ull << i) - 1ull));
            const int q = g + kGroups * k;
            const int ent = q * kRowsPerWG + r;
            tab[pre[k] + r] = make_int2(p.listed ? p.lslot[ent] : q + p.nq * i, ent);
        }
    }
    __syncthreads();
    // this thread's share of every step: down chunk (neuron ln, chunk lc) and
    // a (neuron ln, token lc)
    const int ln = tid / kTile, lc = tid % kTile;
    const int chunk = s * (kSliceOut / 8) + lc;        // chunk of the down column
    const bool cin = chunk < p.cd;
    const u32x4 *dbase = p.bundles + p.dn_off + (cin ? chunk : 0);
    const bool tok_a = lc < p.B;
    const int nst = (ng + kFc2K - 1) / kFc2K;
    u32x4 rv[kSteps];
    float ra[kSteps];
    auto load_step = [&](int st, u32x4 &v, float &a) {
        const int e = st * kFc2K + ln;
        const bool in = st < nst && e < ng;
        const int2 te = tab[in ? e : 0];
        v = (in && cin) ? dbase[(size_t)te.x * p.bstride] : u32x4{0u, 0u, 0u, 0u};
        a = (in && tok_a) ? p.la[(size_t)te.y * p.max_batch + lc] : 0.0f;
    };
    auto stage = [&](int buf, const u32x4 &v, float a) {
        *reinterpret_cast<u32x4 *>(&wl[buf][ln * kWPitch + 8 * lc]) = v;
        al[buf][lc * kAPitch + ln] = (_Float16)a;
    };
    const int gk = lane >> 5, col = lane & 31;
    const int jw = kTile * wave + col;                 // output column within the slice
    f32x16 acc = zero16();
    if (ng > 0) {
#pragma unroll
        for (int u = 0; u < kSteps; ++u) load_step(u, rv[u], ra[u]);
        stage(0, rv[0], ra[0]);
        load_step(kSteps, rv[0], ra[0]);
        __syncthreads();
        for (int st0 = 0; st0 < nst; st0 += kSteps) {
#pragma unroll
            for (int u = 0; u < kSteps; ++u) {
                const int st = st0 + u;
                if (st < nst) {
                    const int nu = (u + 1) % kSteps;
                    if (st + 1 < nst) {
                        stage((st + 1) & 1, rv[nu], ra[nu]);
                        load_step(st + 1 + kSteps, rv[nu], ra[nu]);
                    }
                    const int buf = st & 1;
                    h8 av, bv;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        av[j] = al[buf][col * kAPitch + 8 * gk + j];
                        bv[j] = wl[buf][(8 * gk + j) * kWPitch + jw];
                    }
                    acc = mfma(av, bv, acc);
                    __syncthreads();
                }
            }
        }
    }
    // group tile -> partial; the last group at this slice reduces
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int t = acc_row(i, lane);
        const int m = kSliceOut * s + jw;
        if (t < p.B && m < p.d) p.partial[((size_t)g * p.B + t) * p.d + m] = acc[i];
    }
    if (!arrive_last(p.arrive + s, (unsigned)kGroups, &last_lds)) return;
    for (int idx = tid; idx < p.B * kSliceOut; idx += kThreads) {
        const int t = idx / kSliceOut, m = kSliceOut * s + idx % kSliceOut;
        if (m >= p.d) continue;
        float sum = 0.0f;
#pragma unroll
        for (int gg = 0; gg < kGroups; ++gg) sum += p.partial[((size_t)gg * p.B + t) * p.d + m];
        sum += p.b2[m];
        if (p.resid) sum += p.resid[(size_t)t * p.d + m];
        p.y[(size_t)t * p.d + m] = sum;
    }
}

inline hipEvent_t ev_start(const Trace *tr, int k) { return tr ? tr->ev[2 * k] : nullptr; }
inline hipEvent_t ev_stop(const Trace *tr, int k) { return tr ? tr->ev[2 * k + 1] : nullptr; }
#define ASF_LAUNCH(KID, F, GRID, BLK, ...) \
    hipExtLaunchKernelGGL(F, GRID, BLK, 0, s, ev_start(tr, KID), ev_stop(tr, KID), 0, __VA_ARGS__)

}  // namespace

// split of the predictor's k over workgroups: the largest power of two <= 8
// with d a multiple of 128 * KS (every wave then takes a multiple of 16 k)
int pred_mm_splits(int d) {
    int ks = 8;
    while (ks > 1 && d % (128 * ks) != 0) ks >>= 1;
    return ks;
}

hipError_t launch_pred_mm(const LayerView &L, const float *x, int B, const Trace *tr,
                          hipStream_t s) {
    const int mt = (L.H + kTile - 1) / kTile, ks = pred_mm_splits(L.d);
    ASF_LAUNCH(ASF_K_PRED_L1, k_pred_mm, dim3(mt * ks), dim3(kThreads), (const u32x4 *)L.p1, L.c1,
               x, B, L.d, L.H, ks, L.pred_part, L.pred_arrive, L.h);
    return hipGetLastError();
}

hipError_t launch_score_mm(const LayerView &L, int B, const Trace *tr, hipStream_t s) {
    ASF_LAUNCH(ASF_K_SCORE, k_score_mm, dim3(L.nq), dim3(kThreads), (const u32x4 *)L.p2, L.c2,
               L.h, B, L.H, L.f, L.threshold, L.wbits, L.ubits);
    return hipGetLastError();
}

hipError_t launch_fc1_mm(const LayerView &L, const float *x, int B, int mode, const int32_t *ids,
                         const int32_t *n_ids, const Trace *tr, hipStream_t s) {
    Fc1MmParams p;
    p.bundles = (const u32x4 *)L.bundles;
    p.bstride = (size_t)L.nmat * L.cd;
    p.cd = L.cd;
    p.b1 = L.b1;
    p.x = x;
    p.B = B;
    p.d = L.d;
    p.f = L.f;
    p.mode = mode;
    p.ubits = L.ubits;
    p.ids = ids;
    p.n_ids = n_ids;
    p.inv = L.inv;
    p.vbits = L.vbits;
    p.lslot = L.lslot;
    p.la = L.la;
    p.max_batch = L.max_batch;
    if (L.gated) ASF_LAUNCH(ASF_K_FC1, k_fc1_mm<true>, dim3(L.nq), dim3(kThreads), p);
    else ASF_LAUNCH(ASF_K_FC1, k_fc1_mm<false>, dim3(L.nq), dim3(kThreads), p);
    return hipGetLastError();
}

hipError_t launch_fc2_mm(const LayerView &L, int B, bool listed, const float *resid, float *y,
                         const Trace *tr, hipStream_t s) {
    Fc2MmParams p;
    p.bundles = (const u32x4 *)L.bundles;
    p.bstride = (size_t)L.nmat * L.cd;
    p.dn_off = (L.nmat - 1) * L.cd;
    p.cd = L.cd;
    p.vbits = L.vbits;
    p.lslot = L.lslot;
    p.listed = listed ? 1 : 0;
    p.la = L.la;
    p.max_batch = L.max_batch;
    p.nq = L.nq;
    p.d = L.d;
    p.B = B;
    p.b2 = L.b2;
    p.resid = resid;
    p.y = y;
    p.partial = L.partial;
    p.arrive = L.arrive;
    const int nslice = (L.d + kSliceOut - 1) / kSliceOut;
    ASF_LAUNCH(ASF_K_FC2, k_fc2_mm, dim3(nslice * kGroups), dim3(kThreads), p);
    return hipGetLastError();
}

}  // namespace asf
