// asf_kernels.hip -- gfx950 kernels of the activation-sparse FFN decode path
// (vector form; the batched matrix-core form is asf_batched.hip).
//
// A single-token decode step of one layer is three kernels; the kernel
// boundaries are the grid-wide synchronisation points (on MI355X a boundary
// costs ~1.7 us, less than any in-kernel grid barrier):
//
//   k_pred1      h = ReLU(P1 x + c1)                           dense GEMV
//   k_score1     per owner workgroup q (slots q, q+nq, ...):
//                s = P2 h + c2, bit = s > theta                its 64 P2 rows
//                FC1 of its predicted neurons:                 their up rows
//                a = ReLU(W_up[slot] . x + b1) (or the gated
//                form), listed with their slots
//                FC2 of the same neurons into one fp32 row     their down
//                of d outputs: sum over them of a * column     columns
//   k_fc2_sum    y = b2 (+ residual) + sum over owners of their rows, in
//                owner order
//
// The owner split balances FC1/FC2 without a global prefix sum: with a
// hot-first neuron table, owner q holds ranks q, q+nq, q+2nq, ..., so every
// owner gets the same mix of always-on and rarely-on neurons.  The two
// hottest slots of each owner have their up rows loaded before scoring,
// overlapping the P2 stream; each is used only if that neuron is predicted
// active.
//
// The other entry points use the same building blocks: FC1 over a set
// (k_fc1_1 for one token, k_fc1 for token chunks of 4) and the grouped FC2
// (k_fc2: 16 output slices x 16 neuron groups, the last group at a slice
// sums the partials in fixed order).  The look-ahead stack runs two of the
// per-workgroup bodies in one grid (k_ffn1_pred1, k_score1_fc2sum), so a
// layer takes two launches and the next layer's predictor fills the tails.
//
// Weight reads are whole 16-byte chunks of contiguous rows (a wave load
// instruction covers 1 KiB); an active neuron's up row and down column sit in
// one bundle ("LLM模型之PowerInfer1.0", "其他" question 3: load the active
// columns of the down projection contiguously, skip the inactive ones).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "asf_internal.h"

#include <utility>

namespace asf {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = kThreads / 64;
constexpr int kL2Rows = kRowsPerWG / kWaves;  // predictor layer-2 rows per wave (8)
constexpr int kFc2Batch = 8;                  // FC2 entries in flight per thread
constexpr int kSpecRows = 2;                  // FC1 rows loaded before scoring, per owner
constexpr int kMaxProducers = kMaxFfn / kRowsPerWG / kGroups + 1;

// elements per 16-byte chunk: 8 binary16 or 4 binary32
template <int WT> struct Elt { static constexpr int E = WT ? 8 : 4; };

template <int WT>
__device__ __forceinline__ void unpack(const u32x4 c, float *v) {
    if constexpr (WT == 1) {
        f16x8 h = __builtin_bit_cast(f16x8, c);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (float)h[e];
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(c[e]);
    }
}

template <int E>
__device__ __forceinline__ void load_f32(const float *p, float *v) {
    const float4 *q = reinterpret_cast<const float4 *>(p);
#pragma unroll
    for (int k = 0; k < E / 4; ++k) {
        float4 t = q[k];
        v[4 * k + 0] = t.x;
        v[4 * k + 1] = t.y;
        v[4 * k + 2] = t.z;
        v[4 * k + 3] = t.w;
    }
}

// v of a neighbouring lane through a DPP source modifier (CTRL: the DPP
// control, all rows and banks enabled; every source lane lies inside the
// same 16-lane row, so no lane reads outside the wave)
template <int CTRL> __device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float lane_f(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// Sum over the 64 lanes of a wave (every lane active), the same bits in
// every lane: inside each 16-lane row, DPP adds of lane pairs (quad_perm
// 1,0,3,2), quads (2,3,0,1), half-rows (row_half_mirror) and rows
// (row_mirror) leave the row's sum in each of its lanes; the four row sums,
// read from lanes 0, 16, 32 and 48, are added as (r0 + r1) + (r2 + r3).
// Four dependent ALU steps and four lane reads instead of six cross-lane
// shuffles through the LDS crossbar.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    v += dpp_f<0x140>(v);
    return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

// Sums eight per-lane values v[0..7] (one per row) over the 64 lanes of a
// wave at once: three halving exchanges (lane bit 5, 4, 3 choose which half
// of the remaining rows a lane keeps) leave lane L with row (L >> 3) & 7
// summed over 8 lanes, and three butterfly steps finish the sum over the 8
// lanes holding that row.  Ten shuffles instead of 6 per row.
__device__ __forceinline__ float rows8_sum(const float (&v)[8], int lane) {
    float a[4], b[2];
    const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float send = b5 ? v[k] : v[4 + k], keep = b5 ? v[4 + k] : v[k];
        a[k] = keep + __shfl_xor(send, 32, 64);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const float send = b4 ? a[k] : a[2 + k], keep = b4 ? a[2 + k] : a[k];
        b[k] = keep + __shfl_xor(send, 16, 64);
    }
    float c;
    {
        const float send = b3 ? b[0] : b[1], keep = b3 ? b[1] : b[0];
        c = keep + __shfl_xor(send, 8, 64);
    }
    c += __shfl_xor(c, 4, 64);
    c += __shfl_xor(c, 2, 64);
    c += __shfl_xor(c, 1, 64);
    return c;
}

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// Buffer loads (gfx9 raw buffer instructions): the resource bounds the
// access to [base, base + bytes); a 16-byte load at an offset past the bound
// returns zeros without a memory access.  Loads that a wave may or may not
// need are issued unconditionally this way, so the count of loads in flight
// does not depend on data and the compiler's waits stay exact.  The base and
// bound must be wave-uniform (they go to scalar registers).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kBufWord3 = 0x00020000;   // descriptor word 3: 32-bit data format

__device__ __forceinline__ rsrc_t buf_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kBufWord3);
}

__device__ __forceinline__ u32x4 buf_load(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
}

// a wave-uniform 64-bit value (e.g. an owner word read from LDS) moved to
// scalar registers
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// ---------------------------------------------------------------- layout
// dst row of slot r: r, or with owner_major = nq > 0 the row q*64 + i of
// slot r = q + nq*i (each owner's 64 rows contiguous)
__global__ void k_perm_rows(const u32x4 *__restrict__ src, int C, const int32_t *__restrict__ perm,
                            int nrows, u32x4 *__restrict__ dst, size_t dstride, size_t doff,
                            int owner_major) {
    const size_t total = (size_t)nrows * C;
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * blockDim.x) {
        const int r = (int)(idx / C), c = (int)(idx % C);
        int sr = perm ? perm[r] : r;
        if ((unsigned)sr >= (unsigned)nrows) sr = r;
        const int dr = owner_major > 0 ? (r % owner_major) * kRowsPerWG + r / owner_major : r;
        dst[(size_t)dr * dstride + doff + c] = src[(size_t)sr * C + c];
    }
}

template <typename T>
__global__ __launch_bounds__(256) void k_transpose_perm(const T *__restrict__ wd, int d, int f,
                                                        const int32_t *__restrict__ inv,
                                                        T *__restrict__ bundles, size_t bstride,
                                                        size_t doff) {
    __shared__ T tile[64][65];
    const int i0 = blockIdx.x * 64, m0 = blockIdx.y * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int r = ty; r < 64; r += 4) {
        const int m = m0 + r, i = i0 + tx;
        tile[r][tx] = (m < d && i < f) ? wd[(size_t)m * f + i] : T(0);
    }
    __syncthreads();
    for (int r = ty; r < 64; r += 4) {
        const int i = i0 + r, m = m0 + tx;
        if (i < f && m < d) {
            int s = inv[i];
            if ((unsigned)s >= (unsigned)f) s = i;
            bundles[(size_t)s * bstride + doff + m] = tile[tx][r];
        }
    }
}

// One-token layout of predictor layer 2, k-major: row k holds, for every
// owner q, the 64-entry segment of hidden unit k: (k, q, i) = entry k of
// the P2 row of slot q + nq*i (original id perm[slot]); zero past f.  One
// workgroup per (owner, 64 hidden units), through LDS.
template <typename T>
__global__ __launch_bounds__(256) void k_p2_kmajor(const T *__restrict__ p2, int H, int f, int nq,
                                                   const int32_t *__restrict__ perm,
                                                   T *__restrict__ dst) {
    __shared__ T tile[kRowsPerWG][65];
    const int q = blockIdx.x, k0 = blockIdx.y * 64;
    for (int e = threadIdx.x; e < kRowsPerWG * 64; e += 256) {
        const int i = e / 64, kk = e % 64;
        const int slot = q + nq * i, k = k0 + kk;
        tile[i][kk] = (slot < f && k < H) ? p2[(size_t)perm[slot] * H + k] : (T)0;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < kRowsPerWG * 64; e += 256) {
        const int kk = e / kRowsPerWG, i = e % kRowsPerWG;
        const int k = k0 + kk;
        if (k < H) dst[((size_t)k * nq + q) * kRowsPerWG + i] = tile[i][kk];
    }
}

__global__ void k_invert(const int32_t *__restrict__ perm, int f, int32_t *__restrict__ inv) {
    for (int s = blockIdx.x * blockDim.x + threadIdx.x; s < f; s += gridDim.x * blockDim.x) {
        int id = perm ? perm[s] : s;
        if ((unsigned)id < (unsigned)f) inv[id] = s;
    }
}

__global__ void k_fill_identity(int32_t *__restrict__ v, int n) {
    for (int s = blockIdx.x * blockDim.x + threadIdx.x; s < n; s += gridDim.x * blockDim.x) v[s] = s;
}

__global__ void k_gather_f32(const float *__restrict__ src, const int32_t *__restrict__ perm, int n,
                             float *__restrict__ dst) {
    for (int s = blockIdx.x * blockDim.x + threadIdx.x; s < n; s += gridDim.x * blockDim.x) {
        int id = perm ? perm[s] : s;
        if ((unsigned)id >= (unsigned)n) id = s;
        dst[s] = src ? src[id] : 0.0f;
    }
}

// ---------------------------------------------------------------- predictor layer 1
// WPR waves share one row of P1 (wave part p of row r takes chunks p*64 + lane
// + 64*WPR*i); the WPR wave sums are added in part order, then c1, then ReLU.
template <int WT, int CPL, int BT>
__global__ __launch_bounds__(kThreads) void k_pred_l1(const u32x4 *__restrict__ P1,
                                                      const float *__restrict__ c1,
                                                      const float *__restrict__ x, int B, int d,
                                                      int H, int wpr, float *__restrict__ h) {
    constexpr int E = Elt<WT>::E;
    __shared__ float red[kWaves][BT];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rpw = kWaves / wpr;
    const int row = blockIdx.x * rpw + wave / wpr, part = wave % wpr;
    const int C = d / E;
    const bool live = row < H;
    // every load is issued unconditionally from a clamped address, so all of
    // them are in flight before the first wait; out-of-range chunks are
    // zeroed when used
    const int rowc = live ? row : H - 1;
    u32x4 w[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = part * 64 + lane + 64 * wpr * i;
        w[i] = P1[(size_t)rowc * C + (c < C ? c : C - 1)];
    }
    float xv[BT][CPL][E];
    auto load_x = [&](int b0) {
#pragma unroll
        for (int t = 0; t < BT; ++t)
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = part * 64 + lane + 64 * wpr * i;
                const int tt = (BT == 1 || b0 + t < B) ? b0 + t : b0;
                load_f32<E>(x + (size_t)tt * d + (size_t)(c < C ? c : C - 1) * E, xv[t][i]);
            }
    };
    load_x(0);
    for (int b0 = 0; b0 < B; b0 += BT) {
        float acc[BT];
#pragma unroll
        for (int t = 0; t < BT; ++t) acc[t] = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = part * 64 + lane + 64 * wpr * i;
            if (live && c < C) {
                float wv[E];
                unpack<WT>(w[i], wv);
#pragma unroll
                for (int t = 0; t < BT; ++t)
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[t] = fmaf(wv[e], xv[t][i][e], acc[t]);
            }
        }
        if (b0 + BT < B) load_x(b0 + BT);
#pragma unroll
        for (int t = 0; t < BT; ++t) {
            const float sum = wave_sum(acc[t]);
            if (lane == 0) red[wave][t] = sum;
        }
        __syncthreads();
        if ((int)threadIdx.x < rpw * BT) {
            const int rl = threadIdx.x / BT, t = threadIdx.x % BT;
            const int r = blockIdx.x * rpw + rl;
            if (r < H && (BT == 1 || b0 + t < B)) {
                float sum = 0.0f;
                for (int p = 0; p < wpr; ++p) sum += red[rl * wpr + p][t];
                h[(size_t)(b0 + t) * H + r] = fmaxf(sum + c1[r], 0.0f);
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------- single-token staging
// The B = 1 kernels stage x (and h) in LDS once per workgroup; every wave reads
// the chunk of x it needs from LDS right before the FMAs, so registers hold
// only weight chunks and partial sums (no spills up to d = 8192 fp16).
constexpr int kMaxDLds = 8192;   // floats of x (a d row is at most 16 KiB of weights)
constexpr int kMaxHLds = 2048;   // floats of h

// Each thread loads its float4s of a length-n fp32 vector (n % 4 == 0,
// n <= 4 * kThreads * N4) from clamped addresses, then stores them to LDS.
template <int N4>
__device__ __forceinline__ void stage_load(const float *__restrict__ src, int n, float4 (&v)[N4]) {
    const float4 *s4 = reinterpret_cast<const float4 *>(src);
    const int n4 = n / 4;
#pragma unroll
    for (int i = 0; i < N4; ++i) {
        const int idx = (int)threadIdx.x + kThreads * i;
        v[i] = s4[idx < n4 ? idx : n4 - 1];
    }
}

// Every thread stores (no guard: the LDS array holds N4 * kThreads float4,
// and places past n get copies of the last float4, never read), so the
// staging loads stay where they were issued instead of sinking into a
// guarded store behind a full wait.
// (a pack expansion rather than a loop: a loop the compiler leaves rolled
// indexes v at run time, which puts v in scratch memory)
template <int N4, int NF, size_t... I>
__device__ __forceinline__ void stage_store_i(float (&dst)[NF], const float4 (&v)[N4],
                                              std::index_sequence<I...>) {
    float4 *d4 = reinterpret_cast<float4 *>(dst);
    ((d4[(int)threadIdx.x + kThreads * (int)I] = v[I]), ...);
}

template <int N4, int NF>
__device__ __forceinline__ void stage_store(float (&dst)[NF], const float4 (&v)[N4]) {
    static_assert(NF >= N4 * 4 * kThreads, "LDS staging array too small");
    stage_store_i(dst, v, std::make_index_sequence<N4>{});
}

// acc += chunk c of a weight row (in registers) . chunk c of an LDS vector
template <int WT>
__device__ __forceinline__ float dot_chunk_lds(const u32x4 w, const float *vs, int c, float acc) {
    constexpr int E = Elt<WT>::E;
    float wv[E];
    unpack<WT>(w, wv);
    const float4 *v4 = reinterpret_cast<const float4 *>(vs + c * E);
#pragma unroll
    for (int k = 0; k < E / 4; ++k) {
        const float4 t = v4[k];
        acc = fmaf(wv[4 * k + 0], t.x, acc);
        acc = fmaf(wv[4 * k + 1], t.y, acc);
        acc = fmaf(wv[4 * k + 2], t.z, acc);
        acc = fmaf(wv[4 * k + 3], t.w, acc);
    }
    return acc;
}

// Predictor layer 1 for one token, workgroup `blk`: WPR waves share a row of
// P1 (wave part p takes chunks p*64 + lane + 64*WPR*i, i < kPred1Cpl, WPR the
// smallest power of two that covers the row so), with the x chunks loaded
// beside the weight chunks.  Sums: per lane in chunk order, butterfly over
// the wave, then the parts in order, then c1, then ReLU.
constexpr int kPred1Cpl = 4;

struct Pred1Args {
    const u32x4 *P1;
    const float *c1;
    const float *x;
    int d, H, wpr;
    float *h;
};

template <int WT>
__device__ __forceinline__ void pred1_block(const Pred1Args &a, int blk) {
    constexpr int E = Elt<WT>::E;
    constexpr int CPL = kPred1Cpl;
    __shared__ float red[kWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wpr = a.wpr, H = a.H;
    const int rpw = kWaves / wpr;
    const int row = blk * rpw + wave / wpr, part = wave % wpr;
    const int C = a.d / E;
    const bool live = row < H;
    const int rowc = live ? row : H - 1;
    // the bias of the row this thread finishes (threads < rpw), loaded early
    const int rfin = blk * rpw + (int)threadIdx.x;
    const float c1v = a.c1[rfin < H ? rfin : H - 1];
    u32x4 w[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = part * 64 + lane + 64 * wpr * i;
        w[i] = a.P1[(size_t)rowc * C + (c < C ? c : C - 1)];
    }
    float xr[CPL][E];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = part * 64 + lane + 64 * wpr * i;
        load_f32<E>(a.x + (size_t)(c < C ? c : C - 1) * E, xr[i]);
    }
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = part * 64 + lane + 64 * wpr * i;
        if (live && c < C) {
            float wv[E];
            unpack<WT>(w[i], wv);
#pragma unroll
            for (int e = 0; e < E; ++e) acc = fmaf(wv[e], xr[i][e], acc);
        }
    }
    const float sum = wave_sum(acc);
    if (lane == 0) red[wave] = sum;
    __syncthreads();
    if ((int)threadIdx.x < rpw) {
        const int r = blk * rpw + threadIdx.x;
        if (r < H) {
            float t = 0.0f;
            for (int pp = 0; pp < wpr; ++pp) t += red[threadIdx.x * wpr + pp];
            a.h[r] = fmaxf(t + c1v, 0.0f);
        }
    }
}

// The same rows with x staged in LDS once per workgroup: each thread's
// global loads are its weight chunks and one share of x, instead of the x
// chunks of every weight chunk it holds.  Sums as pred1_block.
template <int WT>
__device__ __forceinline__ void pred1_block_lds(const Pred1Args &a, int blk,
                                                float (&xs)[kMaxDLds]) {
    constexpr int CPL = kPred1Cpl;
    __shared__ float red[kWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wpr = a.wpr, H = a.H;
    const int rpw = kWaves / wpr;
    const int row = blk * rpw + wave / wpr, part = wave % wpr;
    const int C = a.d / Elt<WT>::E;
    const bool live = row < H;
    const int rowc = live ? row : H - 1;
    const int rfin = blk * rpw + (int)threadIdx.x;
    const float c1v = a.c1[rfin < H ? rfin : H - 1];
    u32x4 w[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = part * 64 + lane + 64 * wpr * i;
        w[i] = a.P1[(size_t)rowc * C + (c < C ? c : C - 1)];
    }
    float4 xv[4];
    stage_load<4>(a.x, a.d, xv);
    stage_store<4>(xs, xv);
    __syncthreads();
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = part * 64 + lane + 64 * wpr * i;
        if (live && c < C) acc = dot_chunk_lds<WT>(w[i], xs, c, acc);
    }
    const float sum = wave_sum(acc);
    if (lane == 0) red[wave] = sum;
    __syncthreads();
    if ((int)threadIdx.x < rpw) {
        const int r = blk * rpw + threadIdx.x;
        if (r < H) {
            float t = 0.0f;
            for (int pp = 0; pp < wpr; ++pp) t += red[threadIdx.x * wpr + pp];
            a.h[r] = fmaxf(t + c1v, 0.0f);
        }
    }
}

template <int WT>
__global__ __launch_bounds__(kThreads) void k_pred1(Pred1Args a) {
    __shared__ float xs[kMaxDLds];
    pred1_block_lds<WT>(a, blockIdx.x, xs);
}

// Predictor layer 1 for 2..kPred1MaxB tokens (fp16 weights) in the geometry of
// k_pred1: the weight chunks stay in registers while the tokens go by, the
// x chunks of the next token loaded while the current one is summed.  Each
// token's sum is formed exactly as k_pred1 forms it.  Also writes h as fp16
// hi + lo halves (h16: [2][B][H]) for the batched scores and x as fp16 hi +
// lo (x16, pitch dp, lo rows after Bm hi rows) for the batched FC1.

__global__ __launch_bounds__(kThreads) void k_pred1b(Pred1Args a, int B, _Float16 *__restrict__ h16,
                                                     _Float16 *__restrict__ x16, int dp, int Bm) {
    constexpr int CPL = kPred1Cpl;
    __shared__ float red[kPred1MaxB][kWaves];
    // two tokens' x at a time, staged in LDS by the whole workgroup: each
    // thread's global loads are its weight chunks and shares of x, not the x
    // chunks of every weight chunk for every token
    __shared__ float xs[2][kMaxDLds];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wpr = a.wpr, H = a.H, d = a.d;
    const int rpw = kWaves / wpr;
    const int row = blockIdx.x * rpw + wave / wpr, part = wave % wpr;
    const int C = d / 8;
    const bool live = row < H;
    const int rowc = live ? row : H - 1;
    const int rfin = blockIdx.x * rpw + (int)threadIdx.x / kPred1MaxB;
    const float c1v = a.c1[rfin < H ? rfin : H - 1];
    u32x4 w[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = part * 64 + lane + 64 * wpr * i;
        w[i] = a.P1[(size_t)rowc * C + (c < C ? c : C - 1)];
    }
    // tokens t0, t0 + 1 (the second clamped to B - 1) into LDS
    auto stage_pair = [&](int t0) {
        float4 v0[4], v1[4];
        const int t1 = t0 + 1 < B ? t0 + 1 : B - 1;
        stage_load<4>(a.x + (size_t)t0 * d, d, v0);
        stage_load<4>(a.x + (size_t)t1 * d, d, v1);
        stage_store<4>(xs[0], v0);
        stage_store<4>(xs[1], v1);
    };
    auto tok_sum = [&](int t, const float *xt) {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = part * 64 + lane + 64 * wpr * i;
            if (live && c < C) acc = dot_chunk_lds<1>(w[i], xt, c, acc);
        }
        const float sum = wave_sum(acc);
        if (lane == 0) red[t][wave] = sum;
    };
#pragma unroll
    for (int t = 0; t < kPred1MaxB; t += 2) {
        if (t >= B) break;
        if (t > 0) __syncthreads();   // the previous pair is no longer read
        stage_pair(t);
        __syncthreads();
        tok_sum(t, xs[0]);
        if (t + 1 < B) tok_sum(t + 1, xs[1]);
    }
    __syncthreads();
    // thread t finishes row t / kPred1MaxB for token t % kPred1MaxB
    {
        const int rl = threadIdx.x / kPred1MaxB, t = threadIdx.x % kPred1MaxB;
        const int r = blockIdx.x * rpw + rl;
        if (rl < rpw && r < H && t < B) {
            float sum = 0.0f;
            for (int pp = 0; pp < wpr; ++pp) sum += red[t][rl * wpr + pp];
            const float hv = fmaxf(sum + c1v, 0.0f);
            const _Float16 hi = (_Float16)hv;
            a.h[(size_t)t * H + r] = hv;
            h16[(size_t)t * H + r] = hi;
            h16[(size_t)(B + t) * H + r] = (_Float16)(hv - (float)hi);
        }
    }
    // x -> fp16 hi + lo for the batched FC1
    const int n8 = B * d / 8;
    for (int i = blockIdx.x * kThreads + threadIdx.x; i < n8; i += gridDim.x * kThreads)
        x16_chunk(a.x, d, dp, Bm, x16, i);
}

// ---------------------------------------------------------------- predictor layer 2
// Owner q, wave w scores the slots of bits i = 8w .. 8w+7 (slot q + nq*i);
// lane l holds chunks l, l+64, ... of each row.  Loads are unconditional from
// clamped addresses (rows past f read row f-1 and are discarded later), so
// the whole wave's rows are in flight at once.
template <int CPL>
__device__ __forceinline__ void l2_load(const u32x4 *__restrict__ P2, int f, int C, int q, int nq,
                                        int wave, int lane, u32x4 (&w)[kL2Rows][CPL]) {
#pragma unroll
    for (int j = 0; j < kL2Rows; ++j) {
        const int row = q * kRowsPerWG + wave * kL2Rows + j;   // owner-major P2 row
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            w[j][i] = P2[(size_t)row * C + (c < C ? c : C - 1)];
        }
    }
}

// bits[t] bit j set when the score of row j of this wave exceeds theta for
// token b0 + t.  Lane L ends with row r = (L >> 3) & 7 and adds that row's
// bias, loaded per lane.
template <int WT, int CPL, int BT>
__device__ __forceinline__ void l2_bits(const u32x4 (&w)[kL2Rows][CPL],
                                        const float *__restrict__ c2, const float *__restrict__ h,
                                        int b0, int B, int H, int f, int q, int nq, int wave,
                                        float theta, int lane, uint32_t (&bits)[BT]) {
    constexpr int E = Elt<WT>::E;
    const int C = H / E;
    const int r = (lane >> 3) & 7;
    const int slot_r = q + nq * (wave * kL2Rows + r);
    const bool valid_r = slot_r < f;
    const float bias_r = c2[valid_r ? slot_r : f - 1];
    float hv[BT][CPL][E];
#pragma unroll
    for (int t = 0; t < BT; ++t)
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            const int tt = (BT == 1 || b0 + t < B) ? b0 + t : b0;
            load_f32<E>(h + (size_t)tt * H + (size_t)(c < C ? c : C - 1) * E, hv[t][i]);
        }
    float acc[BT][kL2Rows];
#pragma unroll
    for (int t = 0; t < BT; ++t)
#pragma unroll
        for (int j = 0; j < kL2Rows; ++j) acc[t][j] = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        if (lane + 64 * i < C) {
#pragma unroll
            for (int j = 0; j < kL2Rows; ++j) {
                float wv[E];
                unpack<WT>(w[j][i], wv);
#pragma unroll
                for (int t = 0; t < BT; ++t)
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[t][j] = fmaf(wv[e], hv[t][i][e], acc[t][j]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < BT; ++t) {
        const float sc = rows8_sum(acc[t], lane) + bias_r;
        const uint64_t m = __ballot(valid_r && sc > theta);
        uint32_t b = 0;
#pragma unroll
        for (int j = 0; j < kL2Rows; ++j) b |= (uint32_t)((m >> (8 * j)) & 1ull) << j;
        bits[t] = b;
    }
}

// ---------------------------------------------------------------- FC1
struct Fc1Out {
    uint64_t *vbits;
    int32_t *lslot;
    float *la;
    int max_batch;
};

// a for one neuron whose rows (up, and gate when gated) are in registers:
// lane l holds chunks l, l+64, ... (C chunks in all); lane 0 writes a for
// every token to a_out[t].
template <int WT, bool GATED, int CPL>
__device__ __forceinline__ void fc1_neuron(const u32x4 (&wu)[CPL], const u32x4 (&wg)[CPL], int C,
                                           const float *__restrict__ x, int B, int d, float bias,
                                           int lane, float *__restrict__ a_out) {
    constexpr int E = Elt<WT>::E;
    for (int t = 0; t < B; ++t) {
        float au = 0.0f, ag = 0.0f;
        float xv[CPL][E];
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            load_f32<E>(x + (size_t)t * d + (size_t)(c < C ? c : C - 1) * E, xv[i]);
        }
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            if (c < C) {
                float vu[E];
                unpack<WT>(wu[i], vu);
#pragma unroll
                for (int e = 0; e < E; ++e) au = fmaf(vu[e], xv[i][e], au);
                if constexpr (GATED) {
                    float vg[E];
                    unpack<WT>(wg[i], vg);
#pragma unroll
                    for (int e = 0; e < E; ++e) ag = fmaf(vg[e], xv[i][e], ag);
                }
            }
        }
        const float su = wave_sum(au);
        float a;
        if constexpr (GATED) {
            const float sg = wave_sum(ag);
            a = fmaxf(sg + bias, 0.0f) * su;
        } else {
            a = fmaxf(su + bias, 0.0f);
        }
        if (lane == 0) a_out[t] = a;
    }
}

template <bool GATED, int CPL>
__device__ __forceinline__ void load_fc1_rows(const u32x4 *__restrict__ bundles, size_t bstride,
                                              int C, int slot, int lane, u32x4 (&wu)[CPL],
                                              u32x4 (&wg)[CPL]) {
    const u32x4 *bp = bundles + (size_t)slot * bstride;
    constexpr int UP = GATED ? 1 : 0;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        const int cc = c < C ? c : C - 1;
        wu[i] = bp[(size_t)UP * C + cc];
        if constexpr (GATED) wg[i] = bp[cc];
        else wg[i] = zero4();
    }
}

// The same rows through a buffer bounded to the bundle of `slot` (wave-
// uniform); with present false nothing is read and the rows are zero.
template <bool GATED, int CPL>
__device__ __forceinline__ void load_fc1_rows_buf(const u32x4 *__restrict__ bundles,
                                                  size_t bstride, int C, int slot, bool present,
                                                  int lane, u32x4 (&wu)[CPL], u32x4 (&wg)[CPL]) {
    slot = __builtin_amdgcn_readfirstlane(slot);
    const uint32_t bytes = present ? (uint32_t)(16 * bstride) : 0u;
    const rsrc_t rs = buf_rsrc(bundles + (size_t)slot * bstride, bytes);
    constexpr int UP = GATED ? 1 : 0;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        // chunks past the row read past the bound
        wu[i] = buf_load(rs, c < C ? 16u * (UP * C + c) : bytes);
        if constexpr (GATED) wg[i] = buf_load(rs, c < C ? 16u * c : bytes);
        else wg[i] = zero4();
    }
}

// FC1 of owner q over its valid entries (bit i of `valid`, slot slot_of(i)):
// wave w takes entries i = w, w+8, ...; the entry of rank r (r-th set bit)
// is listed at lslot[q][r], la[q][r][0..B).  When spec is set, wave w's
// registers spu/spg already hold the rows of slot_of(w).
template <int WT, bool GATED, int CPL, class SlotOf>
__device__ __forceinline__ void owner_fc1(int q, uint64_t valid, SlotOf slot_of,
                                          const u32x4 *__restrict__ bundles, size_t bstride,
                                          int C, const float *__restrict__ b1,
                                          const float *__restrict__ x, int B, int d, Fc1Out o,
                                          bool spec, const u32x4 (&spu)[CPL],
                                          const u32x4 (&spg)[CPL], int wave, int lane) {
    for (int k = 0; k < kRowsPerWG / kWaves; ++k) {
        const int i = wave + kWaves * k;
        if (!((valid >> i) & 1ull)) continue;
        const int slot = slot_of(i);
        const int rank = __popcll(valid & ((1ull << i) - 1ull));
        u32x4 wu[CPL], wg[CPL];
        if (k == 0 && spec) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                wu[c] = spu[c];
                wg[c] = spg[c];
            }
        } else {
            load_fc1_rows<GATED, CPL>(bundles, bstride, C, slot, lane, wu, wg);
        }
        const float bias = b1[slot];
        const size_t e = (size_t)q * kRowsPerWG + rank;
        fc1_neuron<WT, GATED, CPL>(wu, wg, C, x, B, d, bias, lane, o.la + e * o.max_batch);
        if (lane == 0) o.lslot[e] = slot;
    }
}

struct ScoreParams {
    const u32x4 *p2;
    const void *p2k;  // [nq][H][64] one-token layout of P2 (k-major per owner)
    const float *c2;
    const float *h;
    int B, H, f;
    float theta;
    uint64_t *wbits;  // [B][nq]
    uint64_t *ubits;  // [nq]
    // FC1 (decode-step form)
    const u32x4 *bundles;
    size_t bstride;   // chunks per bundle
    int cd;           // chunks per d row
    const float *b1;
    const float *x;
    int d;
    Fc1Out out;
    // single-token FC2 partial rows: [d/16][nq][16], owner q's sum over its
    // listed neurons of a * (down column), 16 outputs per slice
    int dn_off;       // chunk offset of the down column in a bundle
    float *part1;
    // a caller's list of original ids (one token over a given set)
    const int32_t *ids;
    const int32_t *n_ids;
    const int32_t *inv;
    // one-token step in one launch: predictor layer 1 rows of each owner and
    // the exchange of h between the owners
    const void *p1;       // [H][d]
    const float *c1;      // [H]
    int l1_rows;          // rows of h per owner
    int l1_wpr;           // waves per row
    uint64_t *xch;        // [kXchCopies][xstride]: (epoch << 32) | h bits
    int xstride;
    const unsigned *epoch;
    unsigned *flags;      // bit kFlagXchTimeout: an exchange wait gave up
};

// Owner workgroup q: score its 64 slots for every token, store per-token and
// union owner bits; with FC1, then list its union-active neurons with a.
template <int WT, int CPL2, int BT, bool FC1, bool GATED, int CPL1>
__global__ __launch_bounds__(kThreads) void k_score(ScoreParams p) {
    __shared__ uint32_t bits_lds[BT][kWaves];
    __shared__ uint64_t u_lds;
    const int q = blockIdx.x, nq = gridDim.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    u32x4 w2[kL2Rows][CPL2];
    l2_load<CPL2>(p.p2, p.f, p.H / Elt<WT>::E, q, nq, wave, lane, w2);
    // speculative FC1 rows of the owner's kSpecRows hottest slots (bit i =
    // wave, slot q + nq*wave), in flight while P2 streams
    u32x4 spu[FC1 ? CPL1 : 1], spg[FC1 ? CPL1 : 1];
    const int spec_slot = q + nq * wave;
    const bool spec = FC1 && wave < kSpecRows && spec_slot < p.f;
    if constexpr (FC1) {
        if (spec) load_fc1_rows<GATED, CPL1>(p.bundles, p.bstride, p.cd, spec_slot, lane, spu, spg);
    }
    uint64_t u = 0;
    for (int b0 = 0; b0 < p.B; b0 += BT) {
        uint32_t bits[BT];
        l2_bits<WT, CPL2, BT>(w2, p.c2, p.h, b0, p.B, p.H, p.f, q, nq, wave, p.theta, lane,
                              bits);
        if (lane == 0) {
#pragma unroll
            for (int t = 0; t < BT; ++t) bits_lds[t][wave] = bits[t];
        }
        __syncthreads();
        if (threadIdx.x == 0) {
#pragma unroll
            for (int t = 0; t < BT; ++t) {
                if (BT == 1 || b0 + t < p.B) {
                    uint64_t m = 0;
#pragma unroll
                    for (int w = 0; w < kWaves; ++w) m |= (uint64_t)bits_lds[t][w] << (kL2Rows * w);
                    p.wbits[(size_t)(b0 + t) * nq + q] = m;
                    u |= m;
                }
            }
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        p.ubits[q] = u;
        u_lds = u;
        if (FC1) p.out.vbits[q] = u;
    }
    __syncthreads();
    if constexpr (FC1) {
        auto slot_of = [&](int i) { return q + nq * i; };
        owner_fc1<WT, GATED, CPL1>(q, u_lds, slot_of, p.bundles, p.bstride, p.cd, p.b1, p.x, p.B,
                                   p.d, p.out, spec, spu, spg, wave, lane);
    }
}

struct Fc1Params {
    const u32x4 *bundles;
    size_t bstride;
    int cd;
    const float *b1;
    const float *x;
    int B, d, f;
    int mode;              // 0 union of last prediction, 1 caller ids, 2 all
    const uint64_t *ubits;
    const int32_t *ids;
    const int32_t *n_ids;
    const int32_t *inv;
    Fc1Out out;
};

// FC1 over a neuron set, owner q taking entries q, q+nq, ... (mode 0/2: slot
// q + nq*i; mode 1: caller id number q + nq*i mapped to its slot).
template <int WT, bool GATED, int CPL1>
__global__ __launch_bounds__(kThreads) void k_fc1(Fc1Params p) {
    __shared__ int slot_lds[kRowsPerWG];
    __shared__ uint64_t valid_lds;
    const int q = blockIdx.x, nq = gridDim.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (threadIdx.x < kRowsPerWG) {
        const int i = threadIdx.x;
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
        if (i == 0) valid_lds = b;
    }
    __syncthreads();
    const uint64_t valid = valid_lds;
    if (threadIdx.x == 0) p.out.vbits[q] = valid;
    u32x4 none[CPL1];
#pragma unroll
    for (int c = 0; c < CPL1; ++c) none[c] = zero4();
    auto slot_of = [&](int i) { return slot_lds[i]; };
    owner_fc1<WT, GATED, CPL1>(q, valid, slot_of, p.bundles, p.bstride, p.cd, p.b1, p.x, p.B, p.d,
                               p.out, false, none, none, wave, lane);
}

// ---------------------------------------------------------------- single-token score / FC1
// FC1 of one neuron for one token with x in LDS; returns a (every lane).
template <int WT, bool GATED, int CPL>
__device__ __forceinline__ float fc1_one(const u32x4 (&wu)[CPL], const u32x4 (&wg)[CPL], int C,
                                         const float *xs, float bias, int lane) {
    float au = 0.0f, ag = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        if (c < C) {
            au = dot_chunk_lds<WT>(wu[i], xs, c, au);
            if constexpr (GATED) ag = dot_chunk_lds<WT>(wg[i], xs, c, ag);
        }
    }
    const float su = wave_sum(au);
    if constexpr (GATED) return fmaxf(wave_sum(ag) + bias, 0.0f) * su;
    else return fmaxf(su + bias, 0.0f);
}

// FC1 of owner q's valid entries for one token (x in LDS): wave w takes
// entries i = w + 8k for k >= k0; the entry of rank r (r-th set bit of
// `valid`) is listed at lslot[q][r], la[q][r], and at a_lds[r] when a_lds
// is given.
template <int WT, bool GATED, int CPL>
__device__ __forceinline__ void fc1_entry_1(int q, uint64_t valid, int i, int slot,
                                            const u32x4 (&wu)[CPL], const u32x4 (&wg)[CPL],
                                            int C, float bias, const float *xs, Fc1Out o,
                                            float *a_lds, int lane) {
    const int rank = __popcll(valid & ((1ull << i) - 1ull));
    const float a = fc1_one<WT, GATED, CPL>(wu, wg, C, xs, bias, lane);
    if (lane == 0) {
        const size_t e = (size_t)q * kRowsPerWG + rank;
        o.la[e * o.max_batch] = a;
        o.lslot[e] = slot;
        if (a_lds) a_lds[rank] = a;
    }
}

template <int WT, bool GATED, int CPL, class SlotOf>
__device__ __forceinline__ void owner_fc1_1(int q, uint64_t valid, SlotOf slot_of, int k0,
                                            const u32x4 *__restrict__ bundles, size_t bstride,
                                            int C, const float *__restrict__ b1, const float *xs,
                                            Fc1Out o, float *a_lds, int wave, int lane) {
    for (int k = k0; k < kRowsPerWG / kWaves; ++k) {
        const int i = wave + kWaves * k;
        if (!((valid >> i) & 1ull)) continue;
        const int slot = slot_of(i);
        const float bias = b1[slot];
        u32x4 wu[CPL], wg[CPL];
        load_fc1_rows<GATED, CPL>(bundles, bstride, C, slot, lane, wu, wg);
        fc1_entry_1<WT, GATED, CPL>(q, valid, i, slot, wu, wg, C, bias, xs, o, a_lds, lane);
    }
}

// registers per FC1 row set (up, and gate when gated), in 16-byte chunks
template <bool GATED, int CPL1, bool SPEC = false, bool WIDE = false> struct Fc1Regs {
    static constexpr int chunks = CPL1 * (GATED ? 2 : 1);
    // at most 128 VGPRs (4 waves per SIMD) while the rows fit beside the P2
    // double buffer; more otherwise, and when the hottest rows are held
    // through the scoring phase or more down columns are requested ahead
    // (WIDE; both used when one workgroup per CU covers every owner)
    static constexpr int waves_per_eu = (chunks <= 14 && !SPEC && !WIDE) ? 4 : 2;
};

// Chunks t, t + 512, ... (thread t) of the down columns of the next N
// entries of `m` (ascending bits, slot q + nq*bit); returns m without those
// entries.  Buffer loads bounded to the column: entries past the last one
// (and chunks past the row) read zeros without touching memory.
template <int N, int CPT>
__device__ __forceinline__ uint64_t load_down(u32x4 (&dv)[N][CPT], uint64_t m,
                                              const u32x4 *__restrict__ dn, size_t bstride, int q,
                                              int nq, int cd) {
    m = uniform64(m);
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const bool present = m != 0ull;
        const int i = present ? __builtin_ctzll(m) : 0;
        m &= m - 1ull;
        const rsrc_t rs = buf_rsrc(dn + (size_t)(q + nq * i) * bstride, present ? 16u * cd : 0u);
#pragma unroll
        for (int j = 0; j < CPT; ++j) dv[n][j] = buf_load(rs, 16u * (threadIdx.x + kThreads * j));
    }
    return m;
}

// acc += a[n0 + n] * dv[n] for the entries below cnt, in entry order
template <int WT, int N, int CPT>
__device__ __forceinline__ void fma_down(const u32x4 (&dv)[N][CPT], int n0, int cnt,
                                         const float *a_lds, float (&acc)[CPT][Elt<WT>::E]) {
    constexpr int E = Elt<WT>::E;
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const float a = n0 + n < cnt ? a_lds[(n0 + n) & (kRowsPerWG - 1)] : 0.0f;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            float vd[E];
            unpack<WT>(dv[n][j], vd);
#pragma unroll
            for (int e = 0; e < E; ++e) acc[j][e] = fmaf(a, vd[e], acc[j][e]);
        }
    }
}

// FC1 of owner q's listed neurons (the bits of `valid`, slot q + nq*bit) and
// the owner's FC2 row, one token, x in LDS.  With SPEC, waves below
// kSpecRows already hold the rows (spu, spg) and bias of bit `wave`.
template <int WT, bool GATED, int CPL1, bool SPEC, bool WIDE = false>
__device__ __forceinline__ void owner_ffn1(const ScoreParams &p, int q, int nq, uint64_t valid_in,
                                           const float *xs, float *a_lds,
                                           const u32x4 (&spu)[CPL1], const u32x4 (&spg)[CPL1],
                                           float spec_bias, int wave, int lane) {
    constexpr int E = Elt<WT>::E;
    const uint64_t valid = uniform64(valid_in);
    const int cnt = __popcll(valid);
    // FC2 of this owner's listed neurons: thread t takes chunks t, t + 512
    // of the down columns.  The chunks of the first PF entries (rank
    // order) are requested now, after the FC1 rows, and with a 256-VGPR
    // budget those of the next PFB too; the rest in batches of PF2 once the
    // FC1 rows are no longer held.  PF is cut where the FC1 rows leave no
    // registers under the 128-VGPR cap.
    constexpr int CPT = (CPL1 + 7) / 8;      // d-row chunks per thread
    constexpr int PF2 = 8 / CPT;
    constexpr bool kWide = Fc1Regs<GATED, CPL1, SPEC, WIDE>::waves_per_eu == 2;
    constexpr bool kTight = !kWide && CPT == 2;
    constexpr int PF = kTight ? (CPL1 >= 12 ? 0 : 2) : PF2;   // no spills
    constexpr int PFB = (kWide && Fc1Regs<GATED, CPL1>::chunks + 2 * PF * CPT <= 32) ? PF : 0;
    // FC1 balanced by rank: with SPEC, bit b < kSpecRows (rows held) is
    // wave b's; the other entries, ranked among themselves, go to waves
    // off, off + 1, ... round the 8 waves
    constexpr int off = SPEC ? kSpecRows : 0;
    const uint64_t mr = SPEC ? (valid & ~((1ull << kSpecRows) - 1ull)) : valid;
    const int nr = __popcll(mr);
    int r = (wave - off + kWaves) % kWaves;
    // with room for them, every FC1 row set of the wave (two for up to 16
    // listed neurons when two sets and the down columns in flight fit 48
    // chunks per lane, else one) is requested before the down columns, in
    // one round trip; a row the wave does not have reads nothing
    constexpr int kCh = Fc1Regs<GATED, CPL1>::chunks;
    constexpr int kHeld = (SPEC ? kCh : 0) + (PF + PFB) * CPT;
    constexpr int HR = !kWide ? 0 : kCh <= 8 || kHeld + 2 * kCh <= 48 ? 2
                                  : kHeld + kCh <= 48 ? 1 : 0;
    u32x4 hu[HR > 0 ? HR : 1][CPL1], hg[HR > 0 ? HR : 1][CPL1];
    float hbias[HR > 0 ? HR : 1];
    int hbit[HR > 0 ? HR : 1];
#pragma unroll
    for (int k = 0; k < HR; ++k) {
        const bool has = r + kWaves * k < nr;
        hbit[k] = has ? nth_set_bit(mr, r + kWaves * k) : 0;
        const int slot = q + nq * hbit[k];
        hbias[k] = p.b1[slot < p.f ? slot : p.f - 1];
        load_fc1_rows_buf<GATED, CPL1>(p.bundles, p.bstride, p.cd, slot, has, lane, hu[k], hg[k]);
    }
    const u32x4 *dn = p.bundles + p.dn_off;
    u32x4 dv[PF > 0 ? PF : 1][CPT];
    u32x4 dvb[PFB > 0 ? PFB : 1][CPT];
    uint64_t rest = valid;
    if constexpr (PF > 0) rest = load_down<PF, CPT>(dv, valid, dn, p.bstride, q, nq, p.cd);
    if constexpr (PFB > 0) rest = load_down<PFB, CPT>(dvb, rest, dn, p.bstride, q, nq, p.cd);
    if constexpr (SPEC) {
        if (wave < kSpecRows && ((valid >> wave) & 1ull)) {
            const int slot = q + nq * wave;
            fc1_entry_1<WT, GATED, CPL1>(q, valid, wave, slot, spu, spg, p.cd, spec_bias, xs,
                                         p.out, a_lds, lane);
        }
    }
#pragma unroll
    for (int k = 0; k < HR; ++k) {
        if (r + kWaves * k < nr)
            fc1_entry_1<WT, GATED, CPL1>(q, valid, hbit[k], q + nq * hbit[k], hu[k], hg[k], p.cd,
                                         hbias[k], xs, p.out, a_lds, lane);
    }
    for (r += kWaves * HR; r < nr; r += kWaves) {
        const int i = nth_set_bit(mr, r);
        const int slot = q + nq * i;
        const float bias = p.b1[slot];
        u32x4 wu[CPL1], wg[CPL1];
        load_fc1_rows<GATED, CPL1>(p.bundles, p.bstride, p.cd, slot, lane, wu, wg);
        fc1_entry_1<WT, GATED, CPL1>(q, valid, i, slot, wu, wg, p.cd, bias, xs, p.out, a_lds,
                                     lane);
    }
    __syncthreads();
    float acc2[CPT][E];
#pragma unroll
    for (int j = 0; j < CPT; ++j)
#pragma unroll
        for (int e = 0; e < E; ++e) acc2[j][e] = 0.0f;
    if constexpr (PF > 0) fma_down<WT, PF, CPT>(dv, 0, cnt, a_lds, acc2);
    if constexpr (PFB > 0) fma_down<WT, PFB, CPT>(dvb, PF, cnt, a_lds, acc2);
    for (int n0 = PF + PFB; n0 < cnt; n0 += PF2) {
        u32x4 dv2[PF2][CPT];
        rest = load_down<PF2, CPT>(dv2, rest, dn, p.bstride, q, nq, p.cd);
        fma_down<WT, PF2, CPT>(dv2, n0, cnt, a_lds, acc2);
    }
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int c = threadIdx.x + kThreads * j;
        if (c < p.cd) {
            const int o = c * E;
            float4 *dst = reinterpret_cast<float4 *>(p.part1 + ((size_t)(o >> 4) * nq + q) * 16 + (o & 15));
#pragma unroll
            for (int k = 0; k < E / 4; ++k) {
                const f32x4 v = {acc2[j][4 * k], acc2[j][4 * k + 1], acc2[j][4 * k + 2],
                                 acc2[j][4 * k + 3]};
                __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(dst + k));
            }
        }
    }
}

// Single-token owner workgroup q: scores of its 64 slots, owner bits; with
// FC1, a of its listed neurons and then the owner's FC2 partial row (its
// listed neurons' a times their down columns, added in rank order), which
// k_fc2_sum adds over owners.  The down columns sit right after the up rows
// in each bundle, so every listed neuron costs one contiguous bundle read.
//
// Predictor layer 2 skips the hidden units that ReLU set to zero: they add
// nothing to any score, so only the P2 entries of the nonzero units are read
// (the pages' principle, computing only what a nonzero activation needs,
// applied to the predictor's own ReLU layer; with a ReLU hidden layer about
// half the units are zero for each token).  P2 is stored k-major (p2k,
// [H][nq][64]): hidden unit k is one contiguous run holding every owner's
// 64-entry segment (128 bytes in fp16), so a zero unit is skipped as a
// whole run and the units that are read are read in full by the owners
// together.  The nonzero units are listed in LDS in ascending order; lane l
// of a wave takes chunk l % CPS of segment l / CPS of each load, every
// segment of a round requested before the first is used, units past the
// list read out of the buffer's range (zeros, no memory traffic).  Sums per
// slot: lane order over the wave's segments, a halving exchange over the
// lanes of one chunk position, then the waves in order, then c2.
//
// With at most 128 VGPRs (4 waves per SIMD) two workgroups fit on a CU, so
// up to 512 owners (f <= 32768) run in one round.
constexpr int kSegRound = 16;   // segment loads per wave per round

template <int WT, class After>
__device__ __forceinline__ void score1_p2(const ScoreParams &p, int q, int nq, int n,
                                          const int2 *seg,
                                          float (&part)[kWaves][kRowsPerWG], int wave, int lane,
                                          After after_first_round) {
    constexpr int E = Elt<WT>::E;           // slots per 16-byte chunk
    constexpr int CPS = kRowsPerWG / E;     // chunks per segment: 8 (fp16) or 16 (fp32)
    constexpr int SPI = 64 / CPS;           // segments per wave load: 8 or 4
    constexpr int STEP = kSegRound * kWaves * SPI;
    const uint32_t seg_bytes = kRowsPerWG * (WT ? 2u : 4u);
    const uint32_t all_bytes = (uint32_t)p.H * (uint32_t)nq * seg_bytes;
    const rsrc_t rs = buf_rsrc(p.p2k, all_bytes);
    const uint32_t own = (uint32_t)q * seg_bytes + 16u * (lane % CPS);
    const int sl = lane / CPS, ch = lane % CPS;
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0f;
    u32x4 w[kSegRound];
    float hg[kSegRound];
    auto issue = [&](int g0) {
#pragma unroll
        for (int j = 0; j < kSegRound; ++j) {
            const int g = g0 + (j * kWaves + wave) * SPI + sl;
            const int2 e = seg[g < n ? g : 0];
            hg[j] = g < n ? __int_as_float(e.y) : 0.0f;
            w[j] = buf_load(rs, g < n ? (uint32_t)e.x + own : all_bytes);
        }
    };
    auto consume = [&]() {
#pragma unroll
        for (int j = 0; j < kSegRound; ++j) {
            float wv[E];
            unpack<WT>(w[j], wv);
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] = fmaf(hg[j], wv[e], acc[e]);
        }
    };
    issue(0);
    // the owner's hottest FC1 rows follow the first round of segments
    __builtin_amdgcn_sched_barrier(0);
    after_first_round();
    __builtin_amdgcn_sched_barrier(0);
    consume();
    for (int g0 = STEP; g0 < n; g0 += STEP) {
        issue(g0);
        consume();
    }
    // halving exchange over lane bits 5, 4 (, 3): the lanes of one chunk
    // position hold the same E slots; each step keeps half of them and adds
    // the partner's other half, so every lane ends with one slot
    float v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = acc[e];
    int off = 0;
#pragma unroll
    for (int half = E / 2, b = 32; half >= 1; half /= 2, b /= 2) {
        const bool hi = lane & b;
#pragma unroll
        for (int k = 0; k < half; ++k) {
            const float keep = hi ? v[half + k] : v[k], send = hi ? v[k] : v[half + k];
            v[k] = keep + __shfl_xor(send, b, 64);
        }
        off += hi ? half : 0;
    }
    part[wave][ch * E + off] = v[0];
}

// The one-launch step (FUSED): owner q first computes rows q*R .. q*R+R-1 of
// h = ReLU(P1 x + c1) in k_pred1's geometry (x staged in LDS, WPR waves per
// row, at most two passes of 8 / WPR rows, every P1 chunk requested up front),
// publishes them to kXchCopies copies of the exchange buffer as 64-bit words
// (epoch << 32 | h bits, device-scope stores) and reads all H words of copy
// q % kXchCopies back (device-scope loads) until every word carries this
// call's epoch.  Nothing else is in flight meanwhile: P2 is requested only
// once h is known (its nonzero units decide which P2 runs are read).  Every
// owner must be resident at once (the launcher checks the occupancy); each
// wait is bounded (kSpinMax reads), after which the word is taken as it is
// and kFlagXchTimeout is raised.  The epoch advances once per step, in the
// owner-row sum that follows the launch.
constexpr int kSpinMax = 1 << 16;
constexpr int kXchPause = 16;   // s_sleep units (64 clocks) before the first exchange read
constexpr unsigned kFlagXchTimeout = 8u;

// this owner's P1 chunks: pass ps, row q*R + ps*rpw + wave/wpr (rows past
// R or H read nothing)
template <int CPL>
__device__ __forceinline__ void step1_load_p1(const ScoreParams &p, int q, int wave, int lane,
                                              u32x4 (&w)[2][CPL]) {
    const int H = p.H, R = p.l1_rows, wpr = p.l1_wpr, rpw = kWaves / wpr;
    const int C = p.cd, part = wave % wpr;
    const uint32_t row_bytes = 16u * (uint32_t)C;
    const uint32_t p1_bytes = (uint32_t)H * row_bytes;
    const rsrc_t rs = buf_rsrc(p.p1, p1_bytes);
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
        const int r = ps * rpw + wave / wpr, row = q * R + r;
        const bool live = r < R && row < H;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = part * 64 + lane + 64 * wpr * i;
            w[ps][i] = buf_load(rs, (live && c < C) ? (uint32_t)row * row_bytes + 16u * c : p1_bytes);
        }
    }
}

template <int WT>
__device__ __forceinline__ void step1_h(const ScoreParams &p, int q, const u32x4 (&w)[2][kPred1Cpl],
                                        const float *xs, float *hs, float (&red)[2][kWaves],
                                        unsigned ep, float c1v, int wave, int lane) {
    constexpr int CPL = kPred1Cpl;
    const int H = p.H, R = p.l1_rows, wpr = p.l1_wpr, rpw = kWaves / wpr;
    const int C = p.cd, part = wave % wpr;
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
        if (ps > 0 && R <= rpw) break;   // one pass covers the owner's rows
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = part * 64 + lane + 64 * wpr * i;
            if (c < C) acc = dot_chunk_lds<WT>(w[ps][i], xs, c, acc);
        }
        const float sum = wave_sum(acc);
        if (lane == 0) red[ps][wave] = sum;
    }
    __syncthreads();
    // publish: thread t < R * kXchCopies stores row t % R to copy t / R
    if ((int)threadIdx.x < R * kXchCopies) {
        const int r = (int)threadIdx.x % R, cp = (int)threadIdx.x / R, row = q * R + r;
        if (row < H) {
            const int ps = r / rpw, rl = r % rpw;
            float t = 0.0f;
            for (int pp = 0; pp < wpr; ++pp) t += red[ps][rl * wpr + pp];
            const float hv = fmaxf(t + c1v, 0.0f);
            const uint64_t word = ((uint64_t)ep << 32) | __float_as_uint(hv);
            __hip_atomic_store(p.xch + (size_t)cp * p.xstride + row, word, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // read h back: thread t takes units t, t + 512, ...
    constexpr int NU = kMaxHLds / kThreads;
    uint64_t *src = p.xch + (size_t)(q % kXchCopies) * p.xstride;
    uint64_t v[NU];
    bool wait[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        wait[u] = (int)threadIdx.x + kThreads * u < H;
        v[u] = 0;
    }
    // the other owners publish within a few hundred ns of this one: a short
    // pause lets the first read find nearly all of them
    __builtin_amdgcn_s_sleep(kXchPause);
    for (int it = 0; it < kSpinMax; ++it) {
        bool any = false;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            if (wait[u]) {
                v[u] = __hip_atomic_load(src + threadIdx.x + kThreads * u, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
                wait[u] = (unsigned)(v[u] >> 32) != ep;
                any |= wait[u];
            }
        }
        if (!any) break;
    }
    bool late = false;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int k = (int)threadIdx.x + kThreads * u;
        if (k < H) hs[k] = __uint_as_float((uint32_t)v[u]);
        late |= wait[u];
    }
    if (late) atomicOr(p.flags, kFlagXchTimeout);
}

template <int WT, bool FC1, bool GATED, int CPL1, bool SPEC, bool FUSED = false>
__device__ __forceinline__ void score1_block(const ScoreParams &p, int q, int nq) {
    __shared__ float hs[kMaxHLds];
    __shared__ int2 seg[kMaxHLds];          // nonzero units: (byte offset of the segment, h)
    __shared__ int cnt_lds[kMaxHLds / kThreads][kWaves];
    __shared__ float part[kWaves][kRowsPerWG];
    __shared__ float xs[FC1 ? kMaxDLds : 4];
    __shared__ uint64_t u_lds;
    __shared__ float a_lds[FC1 ? kRowsPerWG : 1];
    constexpr int NU = kMaxHLds / kThreads;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int H = p.H;
    const int slot_l = q + nq * lane;
    float c2v;
    if constexpr (FUSED) {
        // x staged (predictor layer 1 and FC1), this owner's rows of h, the
        // exchange; the score bias of bit lane
        __shared__ float red[2][kWaves];
        // the epoch first, through a vector load (a scalar load would be
        // waited for with the kernel arguments, before any other request);
        // it is needed only at the publication
        const unsigned ep = __hip_atomic_load(p.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        u32x4 w1[2][kPred1Cpl];
        step1_load_p1<kPred1Cpl>(p, q, wave, lane, w1);
        // the layer-1 bias of the row this thread publishes
        const int c1_row = q * p.l1_rows + (int)threadIdx.x % p.l1_rows;
        const float c1v = p.c1[c1_row < H ? c1_row : H - 1];
        __builtin_amdgcn_sched_barrier(0);
        float4 xv[4];
        stage_load<4>(p.x, p.d, xv);
        c2v = p.c2[slot_l < p.f ? slot_l : p.f - 1];
        stage_store<4>(xs, xv);
        __syncthreads();
        step1_h<WT>(p, q, w1, xs, hs, red, ep, c1v, wave, lane);
    } else {
        // staging: h first (the segments depend on it), the score bias of
        // bit lane, x for FC1
        float4 hv[1];
        stage_load<1>(p.h, H, hv);
        c2v = p.c2[slot_l < p.f ? slot_l : p.f - 1];
        float4 xv[FC1 ? 4 : 1];
        if constexpr (FC1) stage_load<4>(p.x, p.d, xv);
        stage_store<1>(hs, hv);
        if constexpr (FC1) stage_store<4>(xs, xv);
    }
    __syncthreads();
    // nonzero hidden units k = t + 512u, listed u-major, then by wave and
    // lane: ascending k
    uint64_t bal[NU];
    bool nz[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int k = (int)threadIdx.x + kThreads * u;
        nz[u] = k < H && hs[k < H ? k : 0] != 0.0f;
        bal[u] = __ballot(nz[u]);
        if (lane == 0) cnt_lds[u][wave] = __popcll(bal[u]);
    }
    __syncthreads();
    int base[NU], n = 0;
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            if (w == wave) base[u] = n;
            n += cnt_lds[u][w];
        }
    // byte offset of unit k's run
    const uint32_t run_bytes = (uint32_t)nq * kRowsPerWG * (WT ? 2u : 4u);
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int k = (int)threadIdx.x + kThreads * u;
        if (nz[u])
            seg[base[u] + __popcll(bal[u] & below)] =
                make_int2((int)((uint32_t)k * run_bytes), __float_as_int(hs[k]));
    }
    __syncthreads();
    // the FC1 rows of the owner's kSpecRows hottest slots (bit wave, slot
    // q + nq*wave), requested behind the first round of P2 segments; waves
    // without one read nothing
    u32x4 spu[FC1 ? CPL1 : 1], spg[FC1 ? CPL1 : 1];
    float spec_bias = 0.0f;
    auto spec_rows = [&]() {
        if constexpr (SPEC) {
            const int spec_slot = q + nq * wave;
            const bool has = wave < kSpecRows && spec_slot < p.f;
            spec_bias = p.b1[spec_slot < p.f ? spec_slot : p.f - 1];
            load_fc1_rows_buf<GATED, CPL1>(p.bundles, p.bstride, p.cd, spec_slot, has, lane, spu,
                                           spg);
        }
    };
    score1_p2<WT>(p, q, nq, n, seg, part, wave, lane, spec_rows);
    __syncthreads();
    if (threadIdx.x < 64) {
        float s = part[0][lane];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) s += part[w][lane];
        s += c2v;
        const uint64_t m = __ballot(slot_l < p.f && s > p.theta);
        if (threadIdx.x == 0) {
            p.wbits[q] = m;
            p.ubits[q] = m;
            if (FC1) p.out.vbits[q] = m;
            u_lds = m;
        }
    }
    __syncthreads();
    if constexpr (FC1)
        owner_ffn1<WT, GATED, CPL1, SPEC>(p, q, nq, u_lds, xs, a_lds, spu, spg, spec_bias, wave,
                                          lane);
}

template <int WT, bool FC1, bool GATED, int CPL1, bool SPEC>
__global__ __launch_bounds__(kThreads) __attribute__((
    amdgpu_waves_per_eu(Fc1Regs<GATED, CPL1, SPEC>::waves_per_eu))) void k_score1(ScoreParams p) {
    score1_block<WT, FC1, GATED, CPL1, SPEC>(p, blockIdx.x, gridDim.x);
}

// the one-token step in one launch: predictor layer 1 in the owners, h
// exchanged between them, then k_score1's body with FC1
template <int WT, bool GATED, int CPL1, bool SPEC>
__global__ __launch_bounds__(kThreads) __attribute__((
    amdgpu_waves_per_eu(Fc1Regs<GATED, CPL1, SPEC>::waves_per_eu))) void k_step1(ScoreParams p) {
    score1_block<WT, true, GATED, CPL1, SPEC, true>(p, blockIdx.x, gridDim.x);
}

// FC1 + FC2 rows of one token over the set of the layer's last prediction
// (its owner words), for the set predicted ahead of time (the look-ahead
// stack) and for asf_sparse_ffn of one token over the last prediction: the
// same per-owner work as k_score1 after its ballot, so the results match
// the decode step bit for bit.
//
// With LIST the set is a caller's list of original ids instead: every owner
// reads the whole list (kListPer ids per thread per pass, all requested at
// once, then their slots through the inverse table) and keeps the ids whose
// slot it owns as its bits; out-of-range ids are skipped, a repeated id sets
// its bit once.
constexpr int kListPer = 4;

// ids j0 + t + 512u (u < kListPer) of thread t (n > 0 ids in the list):
// every request of a pass issued before its first wait; owner q's bits
// ORed into *m
__device__ __forceinline__ void list_pass(const ScoreParams &p, int n, int j0, int q, int nq,
                                          unsigned long long *m) {
    int id[kListPer], sl[kListPer];
#pragma unroll
    for (int u = 0; u < kListPer; ++u) {
        const int e = j0 + (int)threadIdx.x + kThreads * u;
        id[u] = p.ids[e < n ? e : n - 1];
    }
#pragma unroll
    for (int u = 0; u < kListPer; ++u) {
        const unsigned ic = (unsigned)id[u] < (unsigned)p.f ? (unsigned)id[u] : 0u;
        sl[u] = p.inv[ic];
    }
#pragma unroll
    for (int u = 0; u < kListPer; ++u) {
        const int e = j0 + (int)threadIdx.x + kThreads * u;
        if (e < n && (unsigned)id[u] < (unsigned)p.f && sl[u] % nq == q)
            atomicOr(m, 1ull << (sl[u] / nq));
    }
}

template <int WT, bool GATED, int CPL1, bool LIST = false>
__device__ __forceinline__ void ffn1_block(const ScoreParams &p, int q, int nq) {
    __shared__ float xs[kMaxDLds];
    __shared__ float a_lds[kRowsPerWG];
    __shared__ unsigned long long m_lds;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float4 xv[4];
    stage_load<4>(p.x, p.d, xv);
    uint64_t valid = 0;
    u32x4 spu[CPL1], spg[CPL1];
#pragma unroll
    for (int c = 0; c < CPL1; ++c) spu[c] = spg[c] = zero4();
    float spec_bias = 0.0f;
    if constexpr (LIST) {
        int n = *p.n_ids;
        n = n < 0 ? 0 : (n > p.f ? p.f : n);
        // the first pass: ids requested beside x (an empty list reads the
        // inverse table instead, a buffer that exists, and keeps nothing),
        // x to LDS, then the slots
        const int32_t *src = n > 0 ? p.ids : p.inv;
        const int nn = n > 0 ? n : 1;
        int id[kListPer], sl[kListPer];
#pragma unroll
        for (int u = 0; u < kListPer; ++u) {
            const int e = (int)threadIdx.x + kThreads * u;
            id[u] = src[e < nn ? e : nn - 1];
        }
        // the FC1 rows of the owner's two hottest slots, requested while the
        // list is read (with a hot-first table they are in nearly every set)
        {
            const int spec_slot = q + nq * wave;
            spec_bias = p.b1[spec_slot < p.f ? spec_slot : p.f - 1];
            if (wave < kSpecRows && spec_slot < p.f)
                load_fc1_rows<GATED, CPL1>(p.bundles, p.bstride, p.cd, spec_slot, lane, spu, spg);
        }
        if (threadIdx.x == 0) m_lds = 0ull;
        stage_store<4>(xs, xv);
#pragma unroll
        for (int u = 0; u < kListPer; ++u) {
            const unsigned ic = (unsigned)id[u] < (unsigned)p.f ? (unsigned)id[u] : 0u;
            sl[u] = p.inv[ic];
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kListPer; ++u) {
            const int e = (int)threadIdx.x + kThreads * u;
            if (e < n && (unsigned)id[u] < (unsigned)p.f && sl[u] % nq == q)
                atomicOr(&m_lds, 1ull << (sl[u] / nq));
        }
        for (int j0 = kThreads * kListPer; j0 < n; j0 += kThreads * kListPer)
            list_pass(p, n, j0, q, nq, &m_lds);
        __syncthreads();
        valid = m_lds;
    } else {
        valid = p.ubits[q];
        stage_store<4>(xs, xv);
    }
    if (threadIdx.x == 0) p.out.vbits[q] = valid;
    __syncthreads();
    owner_ffn1<WT, GATED, CPL1, LIST, LIST>(p, q, nq, valid, xs, a_lds, spu, spg, spec_bias, wave,
                                            lane);
}

template <int WT, bool GATED, int CPL1, bool LIST>
__global__ __launch_bounds__(kThreads) __attribute__((
    amdgpu_waves_per_eu(Fc1Regs<GATED, CPL1, LIST, LIST>::waves_per_eu))) void k_ffn1(ScoreParams p) {
    ffn1_block<WT, GATED, CPL1, LIST>(p, blockIdx.x, gridDim.x);
}

// ---------------------------------------------------------------- exact mask, single token
// No predictor: owner workgroup q computes the pre-activation z_i + b1 of
// each of its 64 slots from the first row of the bundle (the up row, or the
// gate row when gated), so the set is the true one: z_i + b1 > 0 (strict,
// the FFN's own ReLU decides; "Técnicas dispersas…", section "Viabilidad de
// la sparsidad de activación").  Wave w takes bits w, w+8, ...; the bits'
// ballot is the owner's mask (stored as its owner words, so the list call
// works as after a prediction).  Gated: a = (g + b1) * (up . x) for the
// active bits, their up rows spread over the waves by rank; plain: a = z + b1.
// Then the owner's FC2 row, as in k_score1.  Every mask row is read; only
// the active neurons' down columns (and up rows when gated) are.
template <int WT, bool GATED, int CPL1>
__global__ __launch_bounds__(kThreads) __attribute__((
    amdgpu_waves_per_eu(Fc1Regs<GATED, CPL1>::waves_per_eu))) void k_exact1(ScoreParams p) {
    constexpr int E = Elt<WT>::E;
    __shared__ float xs[kMaxDLds];
    __shared__ float zb[kRowsPerWG];      // z + b1 of bit i (0 past f)
    __shared__ float a_lds[kRowsPerWG];   // a of the active bits, by rank
    __shared__ uint64_t m_lds;
    const int q = blockIdx.x, nq = gridDim.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int C = p.cd;
    float4 xv[4];
    stage_load<4>(p.x, p.d, xv);
    stage_store<4>(xs, xv);
    __syncthreads();
    for (int k = 0; k < kRowsPerWG / kWaves; ++k) {
        const int i = wave + kWaves * k;
        const int slot = q + nq * i;
        const bool ok = slot < p.f;
        const int sl = ok ? slot : p.f - 1;
        const float bias = p.b1[sl];
        const u32x4 *bp = p.bundles + (size_t)sl * p.bstride;   // mask row: chunk 0 of the bundle
        u32x4 w[CPL1];
#pragma unroll
        for (int c = 0; c < CPL1; ++c) {
            const int cc = lane + 64 * c;
            w[c] = bp[cc < C ? cc : C - 1];
        }
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL1; ++c) {
            const int cc = lane + 64 * c;
            if (cc < C) acc = dot_chunk_lds<WT>(w[c], xs, cc, acc);
        }
        const float z = wave_sum(acc) + bias;
        if (lane == 0) zb[i] = ok ? z : 0.0f;
    }
    __syncthreads();
    if (threadIdx.x < 64) {
        const uint64_t m = __ballot(zb[threadIdx.x] > 0.0f);
        if (threadIdx.x == 0) {
            m_lds = m;
            p.wbits[q] = m;
            p.ubits[q] = m;
            p.out.vbits[q] = m;
        }
    }
    __syncthreads();
    if (!p.part1) return;   // mask only (the activation profiler)
    const uint64_t m = m_lds;
    const int cnt = __popcll(m);
    constexpr int CPT = (CPL1 + 7) / 8;      // d-row chunks per thread
    constexpr int PF = 8 / CPT;
    const u32x4 *dn = p.bundles + p.dn_off;
    u32x4 dv[PF][CPT];
    uint64_t rest = load_down<PF, CPT>(dv, m, dn, p.bstride, q, nq, C);
    if constexpr (GATED) {
        for (int r = wave; r < cnt; r += kWaves) {
            const int i = nth_set_bit(m, r);
            const u32x4 *bp = p.bundles + (size_t)(q + nq * i) * p.bstride + C;   // up row
            u32x4 w[CPL1];
#pragma unroll
            for (int c = 0; c < CPL1; ++c) {
                const int cc = lane + 64 * c;
                w[c] = bp[cc < C ? cc : C - 1];
            }
            float acc = 0.0f;
#pragma unroll
            for (int c = 0; c < CPL1; ++c) {
                const int cc = lane + 64 * c;
                if (cc < C) acc = dot_chunk_lds<WT>(w[c], xs, cc, acc);
            }
            const float u = wave_sum(acc);
            if (lane == 0) a_lds[r] = zb[i] * u;
        }
    } else {
        if (threadIdx.x < 64 && ((m >> threadIdx.x) & 1ull))
            a_lds[__popcll(m & ((1ull << threadIdx.x) - 1ull))] = zb[threadIdx.x];
    }
    __syncthreads();
    float acc2[CPT][E];
#pragma unroll
    for (int j = 0; j < CPT; ++j)
#pragma unroll
        for (int e = 0; e < E; ++e) acc2[j][e] = 0.0f;
    fma_down<WT, PF, CPT>(dv, 0, cnt, a_lds, acc2);
    for (int n0 = PF; n0 < cnt; n0 += PF) {
        u32x4 dv2[PF][CPT];
        rest = load_down<PF, CPT>(dv2, rest, dn, p.bstride, q, nq, C);
        fma_down<WT, PF, CPT>(dv2, n0, cnt, a_lds, acc2);
    }
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int c = threadIdx.x + kThreads * j;
        if (c < C) {
            const int o = c * E;
            float4 *dst = reinterpret_cast<float4 *>(p.part1 + ((size_t)(o >> 4) * nq + q) * 16 + (o & 15));
#pragma unroll
            for (int k = 0; k < E / 4; ++k) {
                const f32x4 v = {acc2[j][4 * k], acc2[j][4 * k + 1], acc2[j][4 * k + 2],
                                 acc2[j][4 * k + 3]};
                __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(dst + k));
            }
        }
    }
}

// FC1 over a neuron set for one token (x staged in LDS); modes as k_fc1.
template <int WT, bool GATED, int CPL1>
__global__ __launch_bounds__(kThreads) __attribute__((
    amdgpu_waves_per_eu(Fc1Regs<GATED, CPL1>::waves_per_eu))) void k_fc1_1(Fc1Params p) {
    __shared__ float xs[kMaxDLds];
    __shared__ int slot_lds[kRowsPerWG];
    __shared__ uint64_t valid_lds;
    const int q = blockIdx.x, nq = gridDim.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float4 xv[4];
    stage_load<4>(p.x, p.d, xv);
    if (threadIdx.x < kRowsPerWG) {
        const int i = threadIdx.x;
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
        if (i == 0) valid_lds = b;
    }
    stage_store<4>(xs, xv);
    __syncthreads();
    const uint64_t valid = valid_lds;
    if (threadIdx.x == 0) p.out.vbits[q] = valid;
    auto slot_of = [&](int i) { return slot_lds[i]; };
    owner_fc1_1<WT, GATED, CPL1>(q, valid, slot_of, 0, p.bundles, p.bstride, p.cd, p.b1, xs,
                                 p.out, nullptr, wave, lane);
}

// ---------------------------------------------------------------- FC2
struct Fc2Params {
    const u32x4 *bundles;
    size_t bstride;      // chunks per bundle
    int dn_off;          // chunk offset of the down column in a bundle
    const uint64_t *vbits;
    const int32_t *lslot;
    int listed;          // 0: entry i of owner q is slot q + nq*i; 1: slot from lslot
    const float *la;
    int max_batch;
    int nq, d, B;
    const float *b2;
    const float *resid;
    float *y;
    float *partial;      // [kGroups][B][d]
    unsigned *arrive;    // [kSlices]
};

// Workgroup (slice s, group g): output elements [s*W, (s+1)*W), W = d/16,
// over the neurons listed by owners g, g+16, g+32, ...  The owners' valid-bit
// words are loaded once (in parallel) and prefix-summed in LDS; entry e of
// the group is bit i of owner q with rank r, its slot q + nq*i (or lslot) and
// its activations la[q][r].  Threads form NL neuron lanes x CL chunk lanes
// (CL = W/E); a neuron lane walks entries nl, nl+NL, ... in batches of
// kFc2Batch loads.  The NL lane sums are added in lane order into this
// group's partial; the last group to arrive at the slice adds the 16 partials
// in group order, then b2, then the residual.
template <int WT, int BT>
__global__ __launch_bounds__(kThreads) void k_fc2(Fc2Params p) {
    constexpr int E = Elt<WT>::E;
    __shared__ uint64_t vb[kMaxProducers];
    __shared__ int pre[kMaxProducers + 1];
    __shared__ int2 tab[kMaxProducers * kRowsPerWG];  // entry -> (slot, list index)
    __shared__ float red[kThreads * E];
    __shared__ int last_lds;
    const int s = blockIdx.x % kSlices, g = blockIdx.x / kSlices;
    const int W = p.d / kSlices, CL = W / E, NL = kThreads / CL;
    const int tid = threadIdx.x, nl = tid / CL, cl = tid % CL;
    const bool lane_ok = nl < NL;
    const int np = g < p.nq ? (p.nq - g + kGroups - 1) / kGroups : 0;
    // owner words of this group (np <= 64) and their popcount prefix, by wave 0
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
    // entry table: entry pre[k] + r is the r-th listed neuron of owner
    // g + 16k (bit i of its word); built in one parallel pass
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
    const u32x4 *segbase = p.bundles + p.dn_off + (size_t)s * CL + cl;

    for (int b0 = 0; b0 < p.B; b0 += BT) {
        float yacc[BT][E];
#pragma unroll
        for (int t = 0; t < BT; ++t)
#pragma unroll
            for (int e = 0; e < E; ++e) yacc[t][e] = 0.0f;
        if (lane_ok) {
            for (int e0 = nl; e0 < ng; e0 += NL * kFc2Batch) {
                int slot[kFc2Batch];
                size_t ent[kFc2Batch];
#pragma unroll
                for (int k = 0; k < kFc2Batch; ++k) {
                    const int e = e0 + NL * k;
                    const int2 te = tab[e < ng ? e : ng - 1];
                    slot[k] = te.x;
                    ent[k] = (size_t)te.y;
                }
                // all of the batch's loads back to back (addresses are valid
                // for every k; entries past ng are dropped below)
                u32x4 v[kFc2Batch];
                float a[kFc2Batch][BT];
#pragma unroll
                for (int k = 0; k < kFc2Batch; ++k) {
                    v[k] = segbase[(size_t)slot[k] * p.bstride];
#pragma unroll
                    for (int t = 0; t < BT; ++t) {
                        const int tt = (BT == 1 || b0 + t < p.B) ? b0 + t : b0;
                        a[k][t] = p.la[ent[k] * p.max_batch + tt];
                    }
                }
#pragma unroll
                for (int k = 0; k < kFc2Batch; ++k) {
                    if (e0 + NL * k >= ng) continue;
                    float vd[E];
                    unpack<WT>(v[k], vd);
#pragma unroll
                    for (int t = 0; t < BT; ++t)
#pragma unroll
                        for (int e = 0; e < E; ++e) yacc[t][e] = fmaf(a[k][t], vd[e], yacc[t][e]);
                }
            }
        }
        // sum the neuron lanes (fixed order) into this group's partial
#pragma unroll
        for (int t = 0; t < BT; ++t) {
            if (lane_ok)
#pragma unroll
                for (int e = 0; e < E; ++e) red[nl * W + cl * E + e] = yacc[t][e];
            __syncthreads();
            if (BT == 1 || b0 + t < p.B) {
                for (int w = tid; w < W; w += kThreads) {
                    float sum = 0.0f;
                    for (int l = 0; l < NL; ++l) sum += red[l * W + w];
                    p.partial[((size_t)g * p.B + b0 + t) * p.d + (size_t)s * W + w] = sum;
                }
            }
            __syncthreads();
        }
    }
    // arrive at the slice; the last of the kGroups groups reduces it
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const unsigned old =
            __hip_atomic_fetch_add(p.arrive + s, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = old == (unsigned)(kGroups - 1);
        if (last) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            __hip_atomic_store(p.arrive + s, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        last_lds = last;
    }
    __syncthreads();
    if (last_lds) {
        for (int idx = tid; idx < p.B * W; idx += kThreads) {
            const int b = idx / W, w = idx % W;
            const size_t m = (size_t)s * W + w;
            float sum = 0.0f;
#pragma unroll
            for (int gg = 0; gg < kGroups; ++gg) sum += p.partial[((size_t)gg * p.B + b) * p.d + m];
            sum += p.b2[m];
            if (p.resid) sum += p.resid[(size_t)b * p.d + m];
            p.y[(size_t)b * p.d + m] = sum;
        }
    }
}

// ---------------------------------------------------------------- single-token FC2 sum
// Workgroup s finishes outputs [16s, 16s + 16) from the owners' partial rows
// (slice-major, [d/16][nq][16]): thread t = 4g + c reads float4 column c of
// owners g, g + 128, ... and adds them in that order; the 128 owner lanes
// are then added in a fixed order (32 in sequence, then 4 in a fixed pair
// tree), then b2, then the residual.
constexpr int kSumQ = kMaxFfn / kRowsPerWG / (kThreads / 4);   // owners per thread, at most

struct Fc2SumArgs {
    const float *part;
    int nq;
    const float *b2;
    const float *resid;
    float *y;
    unsigned *epoch;   // advanced by one after a one-launch step (null otherwise)
};

// SQ: owner rows per thread (owners g, g + 128, ... below SQ * 128 >= nq),
// so that no load repeats a row; the sums do not depend on it.
template <int SQ = kSumQ>
__device__ __forceinline__ void fc2_sum_block(const Fc2SumArgs &a, int s) {
    __shared__ float4 red[kThreads];
    const float *__restrict__ part = a.part;
    const int nq = a.nq;
    const float *__restrict__ b2 = a.b2;
    const float *__restrict__ resid = a.resid;
    float *__restrict__ y = a.y;
    const int tid = threadIdx.x;
    const int c = tid & 3, g = tid >> 2;
    const float4 *src = reinterpret_cast<const float4 *>(part + (size_t)s * nq * 16);
    const int o = tid & 15;
    const float bv = b2[16 * s + o];
    const float rv = resid ? resid[16 * s + o] : 0.0f;
    float4 v[SQ];
#pragma unroll
    for (int k = 0; k < SQ; ++k) {
        const int q = g + (kThreads / 4) * k;
        v[k] = src[(size_t)(q < nq ? q : nq - 1) * 4 + c];
    }
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int k = 0; k < SQ; ++k) {
        if (g + (kThreads / 4) * k < nq) {
            acc.x += v[k].x;
            acc.y += v[k].y;
            acc.z += v[k].z;
            acc.w += v[k].w;
        }
    }
    red[tid] = acc;
    __syncthreads();
    if (tid < 64) {
        // lane: output o, quarter u of the 128 owner lanes
        const int u = tid >> 4;
        const float *rf = reinterpret_cast<const float *>(red);
        float sum = 0.0f;
        for (int gg = 32 * u; gg < 32 * u + 32; ++gg) sum += rf[(gg * 4 + (o >> 2)) * 4 + (o & 3)];
        sum += __shfl_down(sum, 16, 64);   // u + (u + 1) for u = 0, 2
        const float hi = __shfl_down(sum, 32, 64);
        if (tid < 16) y[16 * s + o] = (sum + hi) + bv + rv;
    }
}

template <int SQ>
__global__ __launch_bounds__(kThreads) void k_fc2_sum(Fc2SumArgs a) {
    // every owner of the step has finished with the exchange: the next
    // step's words carry the next epoch
    if (a.epoch && blockIdx.x == 0 && threadIdx.x == 0) *a.epoch += 1u;
    fc2_sum_block<SQ>(a, blockIdx.x);
}

// ---------------------------------------------------------------- look-ahead stack on one stream
// With layer l + 1's set predicted from layer l's input, each layer of the
// stack is two launches, each running two kinds of workgroup side by side:
//   k_ffn1_pred1      workgroups below nq: layer l's FC1 + owner FC2 rows
//                     over its set (ffn1_block); the rest: predictor layer 1
//                     of layer l + 1 on the same input (pred1_block)
//   k_score1_fc2sum   workgroups below nq: layer l + 1's scores and owner
//                     words (score1_block); the rest: layer l's output from
//                     its owner rows (fc2_sum_block)
// The long-running kind comes first in each grid and the short one fills
// the CUs as they free up.  Each workgroup does exactly what it does in the
// separate kernels, so results are theirs bit for bit.
template <int WT, bool GATED, int CPL1>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(
    Fc1Regs<GATED, CPL1>::waves_per_eu))) void k_ffn1_pred1(ScoreParams p, int nq, Pred1Args a) {
    if ((int)blockIdx.x < nq) ffn1_block<WT, GATED, CPL1>(p, blockIdx.x, nq);
    else pred1_block<WT>(a, blockIdx.x - nq);
}

template <int WT, int SQ>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(
    Fc1Regs<false, 1>::waves_per_eu))) void k_score1_fc2sum(ScoreParams p, int nq, Fc2SumArgs a) {
    if ((int)blockIdx.x < nq) score1_block<WT, false, false, 1, false>(p, blockIdx.x, nq);
    else fc2_sum_block<SQ>(a, blockIdx.x - nq);
}

// ---------------------------------------------------------------- activation profiler
// counts[perm[s]] += bit s of the owner words of the last single-token pass
// (slot s = q + nq*i is bit i of word q)
__global__ __launch_bounds__(256) void k_count_bits(const uint64_t *__restrict__ words, int f,
                                                    int nq, const int32_t *__restrict__ perm,
                                                    uint32_t *__restrict__ counts) {
    const int sl = blockIdx.x * 256 + threadIdx.x;
    if (sl >= f) return;
    if ((words[sl % nq] >> (sl / nq)) & 1ull) counts[perm[sl]] += 1u;
}

// Hot-first table by exact ranking: key_i = (count descending, id
// ascending); neuron i goes to position #{j : key_j < key_i}, a permutation
// because the keys are distinct.  Keys are compared in LDS tiles.
constexpr int kRankTile = 1024;

__global__ __launch_bounds__(kRankTile) void k_rank_table(const uint32_t *__restrict__ counts,
                                                          int f, int32_t *__restrict__ table) {
    __shared__ uint64_t kt[kRankTile];
    const int i = blockIdx.x * kRankTile + threadIdx.x;
    const uint64_t ki = i < f ? ((uint64_t)(0xffffffffu - counts[i]) << 32) | (uint32_t)i : ~0ull;
    int rank = 0;
    for (int j0 = 0; j0 < f; j0 += kRankTile) {
        const int j = j0 + threadIdx.x;
        kt[threadIdx.x] = j < f ? ((uint64_t)(0xffffffffu - counts[j]) << 32) | (uint32_t)j : ~0ull;
        __syncthreads();
        const int n = f - j0 < kRankTile ? f - j0 : kRankTile;
        for (int t = 0; t < n; ++t) rank += kt[t] < ki;
        __syncthreads();
    }
    if (i < f) table[rank] = i;
}

// ---------------------------------------------------------------- attention-head predictor
// Layer 2 of the attention-head predictor ("LLM模型之PowerInfer1.0", appendix
// "DejaVu": the second two-layer MLP has one output per head of the
// attention block, each a sigmoid select / skip decision; sigmoid(s) > 0.5
// is s > 0, so the decision is taken on the logit against theta).
// Workgroup (w, b) scores heads 64w .. 64w+63 of token b: wave v takes heads
// 64w + 8v + j (j < 8), its rows of Q2 in registers (clamped past nh), h of
// the token staged in LDS and held per lane as in the FFN scores; the 8 row
// sums of a wave meet by rows8_sum, one ballot per wave, and the 64 bits are
// head word w of the token.  With a single word per token the workgroup
// also lists the selected heads (ascending) and their count.
struct HeadArgs {
    const u32x4 *q2;   // [nh][H] row-major
    const float *c2;   // [nh]
    const float *h;    // [B][H]
    int H, nh, words;
    float theta;
    uint64_t *wbits;   // [B][words] (library scratch)
    uint64_t *masks;   // [B][words] or null
    int32_t *heads;    // [B][nh] or null
    int32_t *count;    // [B] or null
};

template <int WT, int CPL2>
__global__ __launch_bounds__(kThreads) void k_head_score(HeadArgs a) {
    constexpr int E = Elt<WT>::E;
    __shared__ float hs[kMaxHLds];
    __shared__ uint32_t bits_lds[kWaves];
    const int w = blockIdx.x, b = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int C2 = a.H / E;
    float4 hv[1];
    stage_load<1>(a.h + (size_t)b * a.H, a.H, hv);
    u32x4 q[kL2Rows][CPL2];
#pragma unroll
    for (int j = 0; j < kL2Rows; ++j) {
        const int r = w * kRowsPerWG + wave * kL2Rows + j;
        const int rc = r < a.nh ? r : a.nh - 1;
#pragma unroll
        for (int i = 0; i < CPL2; ++i) {
            const int c = lane + 64 * i;
            q[j][i] = a.q2[(size_t)rc * C2 + (c < C2 ? c : C2 - 1)];
        }
    }
    const int rr = (lane >> 3) & 7;
    const int head_r = w * kRowsPerWG + wave * kL2Rows + rr;
    const bool valid_r = head_r < a.nh;
    const float bias_r = a.c2[valid_r ? head_r : a.nh - 1];
    stage_store<1>(hs, hv);
    __syncthreads();
    float hr[CPL2][E];
#pragma unroll
    for (int i = 0; i < CPL2; ++i) {
        const int c = lane + 64 * i;
        const float4 *h4 = reinterpret_cast<const float4 *>(hs + (c < C2 ? c : 0) * E);
#pragma unroll
        for (int k = 0; k < E / 4; ++k) {
            const float4 t = h4[k];
            hr[i][4 * k + 0] = t.x;
            hr[i][4 * k + 1] = t.y;
            hr[i][4 * k + 2] = t.z;
            hr[i][4 * k + 3] = t.w;
        }
    }
    float acc[kL2Rows];
#pragma unroll
    for (int j = 0; j < kL2Rows; ++j) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL2; ++i) {
            const int c = lane + 64 * i;
            if (c < C2) {
                float wv[E];
                unpack<WT>(q[j][i], wv);
#pragma unroll
                for (int e = 0; e < E; ++e) s = fmaf(wv[e], hr[i][e], s);
            }
        }
        acc[j] = s;
    }
    const float sc = rows8_sum(acc, lane) + bias_r;
    const uint64_t m = __ballot(valid_r && sc > a.theta);
    if (lane == 0) {
        uint32_t bb = 0;
#pragma unroll
        for (int j = 0; j < kL2Rows; ++j) bb |= (uint32_t)((m >> (8 * j)) & 1ull) << j;
        bits_lds[wave] = bb;
    }
    __syncthreads();
    uint64_t word = 0;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) word |= (uint64_t)bits_lds[v] << (kL2Rows * v);
    if (threadIdx.x == 0) {
        a.wbits[(size_t)b * a.words + w] = word;
        if (a.masks) a.masks[(size_t)b * a.words + w] = word;
        if (a.words == 1 && a.count) a.count[b] = __popcll(word);
    }
    if (a.words == 1 && a.heads && threadIdx.x < 64 && ((word >> threadIdx.x) & 1ull))
        a.heads[(size_t)b * a.nh + __popcll(word & ((1ull << threadIdx.x) - 1ull))] =
            (int)threadIdx.x;
}

// Heads of token b (one 64-lane workgroup per token, words <= 64): lane t
// takes head word t, its popcount is prefix-summed over the wave, and the
// lane lists its word's heads at that offset in ascending order.
__global__ __launch_bounds__(64) void k_head_list(const uint64_t *__restrict__ wbits, int words,
                                                  int nh, int32_t *__restrict__ heads,
                                                  int32_t *__restrict__ count) {
    const int b = blockIdx.x, t = threadIdx.x;
    const uint64_t m = t < words ? wbits[(size_t)b * words + t] : 0ull;
    const int c = __popcll(m);
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (t >= o) incl += v;
    }
    if (heads) {
        int off = incl - c;
        uint64_t u = m;
        while (u) {
            const int j = __builtin_ctzll(u);
            u &= u - 1ull;
            heads[(size_t)b * nh + off++] = 64 * t + j;
        }
    }
    if (count && t == 63) count[b] = incl;
}

// ---------------------------------------------------------------- list
// Slot-ordered outputs from the owner bits, one workgroup per 512 stored
// slots (thread t: slot s0 + t; wave v: slot word s0/64 + v).  Slot s is
// bit s / nq of owner word s % nq.  Every workgroup stages the nq union
// owner words in LDS and counts the union slots below s0 itself (owner q
// holds the slots q + nq*i, so those below s0 are its bits i < ceil((s0 -
// q) / nq)); the table entry of each thread's slot is requested at the start,
// so the ascending list of slots and original ids is written without a
// dependent load.  Per-token masks: the token words of each slot are
// requested together (up to 32 tokens), one ballot per slot word and token.
constexpr int kListSlots = kThreads;

// integer wave sum (every lane active), the DPP pattern of wave_sum
template <int CTRL> __device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ int wave_sum_int(int v) {
    v += dpp_i<0xB1>(v);
    v += dpp_i<0x4E>(v);
    v += dpp_i<0x141>(v);
    v += dpp_i<0x140>(v);
    return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
           __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

// the workgroup sums of two ints (every thread gets both): wave sums, then
// the wave partials in wave order; one barrier
__device__ __forceinline__ int2 block_sum_int2(int a, int b, int2 *red) {
    a = wave_sum_int(a);
    b = wave_sum_int(b);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = make_int2(a, b);
    __syncthreads();
    int2 t = make_int2(0, 0);
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        t.x += red[w].x;
        t.y += red[w].y;
    }
    return t;
}

struct ListArgs {
    const uint64_t *ubits;
    const uint64_t *wbits;
    int B, f, nq, words;
    const int32_t *perm;
    uint64_t *token_masks;
    int32_t *slots;
    int32_t *count;
    int32_t *active_ids;
    int32_t *n_active;
};

template <bool MASKS>
__device__ __forceinline__ void list_block(const ListArgs &a, int blk) {
    __shared__ uint64_t ob[kMaxFfn / 64];
    __shared__ int2 red[kWaves];
    __shared__ int wave_cnt[kWaves];
    const int B = a.B, f = a.f, nq = a.nq, words = a.words;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int s0 = blk * kListSlots;
    const int s = s0 + t;
    const bool in = s < f;
    const int sc = in ? s : f - 1;
    // requests first: the owner words (at most 2 per thread), this slot's
    // table entry, the token words of this slot
    uint64_t o0 = a.ubits[t < nq ? t : nq - 1];
    uint64_t o1 = a.ubits[t + kThreads < nq ? t + kThreads : nq - 1];
    const int32_t id = a.active_ids ? a.perm[sc] : 0;
    uint64_t tw[MASKS ? kMaxBatch : 1];
    if constexpr (MASKS) {
#pragma unroll
        for (int b = 0; b < kMaxBatch; ++b)
            tw[b] = a.wbits[(size_t)(b < B ? b : B - 1) * nq + sc % nq];
    }
    if (t < nq) ob[t] = o0;
    if (t + kThreads < nq) ob[t + kThreads] = o1;
    __syncthreads();
    // union slots below s0, and in all, from the owner words; this thread's
    // slot bit
    int before = 0, total = 0;
    for (int q = t; q < nq; q += kThreads) {
        const uint64_t m = ob[q];
        total += __popcll(m);
        const int k = s0 > q ? (s0 - q + nq - 1) / nq : 0;
        before += __popcll(k >= 64 ? m : (m & ((1ull << k) - 1ull)));
    }
    const bool mine = in && ((ob[sc % nq] >> (sc / nq)) & 1ull);
    const uint64_t bal = __ballot(mine);
    if (lane == 0) wave_cnt[wave] = __popcll(bal);
    const int2 bt = block_sum_int2(before, total, red);
    int off = bt.x + __popcll(bal & ((1ull << lane) - 1ull));
    for (int v = 0; v < wave; ++v) off += wave_cnt[v];
    if (mine) {
        a.slots[off] = s;
        if (a.active_ids) a.active_ids[off] = id;
    }
    if (blk == 0 && t == 0) {
        *a.count = bt.y;
        if (a.n_active) *a.n_active = bt.y;
    }
    if constexpr (MASKS) {
        const int w = s0 / 64 + wave;
        const int sh = sc / nq;
#pragma unroll
        for (int b = 0; b < kMaxBatch; ++b) {
            if (b >= B) break;
            const uint64_t m = __ballot(in && ((tw[b] >> sh) & 1ull));
            if (lane == 0 && w < words) a.token_masks[(size_t)b * words + w] = m;
        }
    }
}

template <bool MASKS>
__global__ __launch_bounds__(kThreads) void k_list(ListArgs a) {
    list_block<MASKS>(a, blockIdx.x);
}

// the owner-row sum of a one-token step (workgroups below nsum) and the
// step's slot-ordered list (the others) in one grid: the list needs only
// the owner words, which the step's launch has finished writing
template <int SQ>
__global__ __launch_bounds__(kThreads) void k_fc2_sum_list(Fc2SumArgs a, int nsum, ListArgs l) {
    if ((int)blockIdx.x < nsum) {
        if (a.epoch && blockIdx.x == 0 && threadIdx.x == 0) *a.epoch += 1u;
        fc2_sum_block<SQ>(a, blockIdx.x);
    } else {
        list_block<false>(l, blockIdx.x - nsum);
    }
}

// ---------------------------------------------------------------- debug-build checks
// Caller content the release build does not validate, for builds with
// ASF_DEBUG: flag bit 1 = an entry out of range, 2 = an entry that appears
// twice (a bitmap of f bits, one atomicOr per entry), 4 = a count outside
// 0 .. f.  The bitmap is cleared by k_zero_u32 first.
__global__ void k_zero_u32(uint32_t *__restrict__ p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
        p[i] = 0u;
}

__global__ void k_check_ids(const int32_t *__restrict__ ids, const int32_t *__restrict__ n_ids,
                            int n_fixed, int f, uint32_t *__restrict__ bitmap,
                            unsigned *__restrict__ flags) {
    int n = n_ids ? *n_ids : n_fixed;
    if (n < 0 || n > f) {
        if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(flags, 4u);
        n = n < 0 ? 0 : f;
    }
    for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < n; e += gridDim.x * blockDim.x) {
        const int id = ids[e];
        if ((unsigned)id >= (unsigned)f) {
            atomicOr(flags, 1u);
            continue;
        }
        const uint32_t bit = 1u << (id & 31);
        if (atomicOr(bitmap + (id >> 5), bit) & bit) atomicOr(flags, 2u);
    }
}

// Traced launches carry their start/stop events on the dispatch packet itself
// (hipExtLaunchKernelGGL), so the events time exactly the kernel.
inline hipEvent_t ev_start(const Trace *tr, int k) { return tr ? tr->ev[2 * k] : nullptr; }
inline hipEvent_t ev_stop(const Trace *tr, int k) { return tr ? tr->ev[2 * k + 1] : nullptr; }
#define ASF_LAUNCH(KID, F, GRID, BLK, ...) \
    hipExtLaunchKernelGGL(F, GRID, BLK, 0, s, ev_start(tr, KID), ev_stop(tr, KID), 0, __VA_ARGS__)

inline int pow2_at_least(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

}  // namespace

// ================================================================ launchers
hipError_t launch_perm_rows(const void *src, int C, const int32_t *perm, int nrows, void *dst,
                            size_t dstride, size_t doff, int owner_major, hipStream_t s) {
    const size_t total = (size_t)nrows * C;
    const int blocks = (int)((total + 255) / 256 < 8192 ? (total + 255) / 256 : 8192);
    hipLaunchKernelGGL(k_perm_rows, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, s,
                       (const u32x4 *)src, C, perm, nrows, (u32x4 *)dst, dstride, doff, owner_major);
    return hipGetLastError();
}

hipError_t launch_transpose_perm(const void *wd, int d, int f, int ws, const int32_t *inv,
                                 void *bundles, size_t bstride, size_t doff, hipStream_t s) {
    dim3 grid((f + 63) / 64, (d + 63) / 64);
    if (ws == 2)
        hipLaunchKernelGGL(k_transpose_perm<uint16_t>, grid, dim3(256), 0, s, (const uint16_t *)wd,
                           d, f, inv, (uint16_t *)bundles, bstride, doff);
    else
        hipLaunchKernelGGL(k_transpose_perm<uint32_t>, grid, dim3(256), 0, s, (const uint32_t *)wd,
                           d, f, inv, (uint32_t *)bundles, bstride, doff);
    return hipGetLastError();
}

hipError_t launch_p2_kmajor(const void *p2, int H, int f, int nq, int ws, const int32_t *perm,
                            void *dst, hipStream_t s) {
    const dim3 grid(nq, (H + 63) / 64);
    if (ws == 2)
        hipLaunchKernelGGL(k_p2_kmajor<uint16_t>, grid, dim3(256), 0, s, (const uint16_t *)p2, H,
                           f, nq, perm, (uint16_t *)dst);
    else
        hipLaunchKernelGGL(k_p2_kmajor<uint32_t>, grid, dim3(256), 0, s, (const uint32_t *)p2, H,
                           f, nq, perm, (uint32_t *)dst);
    return hipGetLastError();
}

hipError_t launch_invert(const int32_t *perm, int f, int32_t *inv, hipStream_t s) {
    const int blocks = (f + 255) / 256;
    hipLaunchKernelGGL(k_fill_identity, dim3(blocks), dim3(256), 0, s, inv, f);
    hipLaunchKernelGGL(k_invert, dim3(blocks), dim3(256), 0, s, perm, f, inv);
    return hipGetLastError();
}

hipError_t launch_gather_f32(const float *src, const int32_t *perm, int n, float *dst,
                             hipStream_t s) {
    hipLaunchKernelGGL(k_gather_f32, dim3((n + 255) / 256), dim3(256), 0, s, src, perm, n, dst);
    return hipGetLastError();
}

// waves per predictor layer-1 row and the resulting chunks per lane (batched
// form), for H rows of cd chunks
static void l1_shape_of(int H, int cd, int *wpr, int *cpl) {
    int w = H >= 2048 ? 1 : pow2_at_least((2048 + H - 1) / H);
    if (w > 8) w = 8;
    while (w < 8 && (cd + 64 * w - 1) / (64 * w) > 8) w *= 2;
    *wpr = w;
    *cpl = pow2_at_least((cd + 64 * w - 1) / (64 * w));
}

static void l1_shape(const LayerView &L, int *wpr, int *cpl) { l1_shape_of(L.H, L.cd, wpr, cpl); }

// single-token form: waves per row = the smallest power of two (<= 8) for
// which a lane takes at most kPred1Cpl chunks; rows per workgroup 8 / that
static int pred1_wpr_of(int cd) {
    int w = 1;
    while (w < kWaves && (cd + 64 * w - 1) / (64 * w) > kPred1Cpl) w *= 2;
    return w;
}

static int pred1_wpr(const LayerView &L) { return pred1_wpr_of(L.cd); }

static Pred1Args pred1_args(const LayerView &L, const float *x) {
    return Pred1Args{(const u32x4 *)L.p1, L.c1, x, L.d, L.H, pred1_wpr(L), L.h};
}

static int pred1_blocks(const LayerView &L) {
    const int rpw = kWaves / pred1_wpr(L);
    return (L.H + rpw - 1) / rpw;
}

hipError_t launch_pred_l1(const LayerView &L, const float *x, int B, const Trace *tr,
                          hipStream_t s) {
    const u32x4 *P1 = (const u32x4 *)L.p1;
    if (B == 1) {
        const dim3 grid(pred1_blocks(L)), blk(kThreads);
        const Pred1Args a = pred1_args(L, x);
        if (L.wtype == ASF_F16) ASF_LAUNCH(ASF_K_PRED_L1, k_pred1<1>, grid, blk, a);
        else ASF_LAUNCH(ASF_K_PRED_L1, k_pred1<0>, grid, blk, a);
        return hipGetLastError();
    }
    if (L.wtype == ASF_F16 && B <= kPred1MaxB) {
        const dim3 grid(pred1_blocks(L)), blk(kThreads);
        ASF_LAUNCH(ASF_K_PRED_L1, k_pred1b, grid, blk, pred1_args(L, x), B, L.h16, L.x16,
                   x16_pitch(L.d), L.max_batch);
        return hipGetLastError();
    }
    if (L.wtype == ASF_F16) return launch_pred_mm(L, x, B, tr, s);
    int wpr, cpl;
    l1_shape(L, &wpr, &cpl);
    const int rpw = kWaves / wpr;
    const dim3 grid((L.H + rpw - 1) / rpw), blk(kThreads);
#define ASF_L1(WT, CPL)                                                                         \
    ASF_LAUNCH(ASF_K_PRED_L1, (k_pred_l1<WT, CPL, 4>), grid, blk, P1, L.c1, x, B, L.d, L.H,    \
               wpr, L.h);
#define ASF_L1W(WT)                   \
    switch (cpl) {                    \
    case 1: ASF_L1(WT, 1) break;      \
    case 2: ASF_L1(WT, 2) break;      \
    case 4: ASF_L1(WT, 4) break;      \
    default: ASF_L1(WT, 8) break;     \
    }
    ASF_L1W(0)   // fp32 weights (fp16 batches went to the forms above)
#undef ASF_L1W
#undef ASF_L1
    return hipGetLastError();
}

// chunks per lane for a d row, rounded up to an instantiated count
static int fc1_cpl(int cd) {
    const int c = (cd + 63) / 64;
    if (c <= 2) return c < 1 ? 1 : c;
    if (c <= 4) return 4;
    if (c <= 8) return 8;
    if (c <= 10) return 10;
    if (c <= 12) return 12;
    if (c <= 14) return 14;
    return 16;
}

static Fc1Out fc1_out(const LayerView &L) { return Fc1Out{L.vbits, L.lslot, L.la, L.max_batch}; }

// parameters of the owner kernels (scores, FC1, the owner FC2 rows) of layer L
static ScoreParams score_params(const LayerView &L, const float *x, int B) {
    ScoreParams p = {};
    p.p2 = (const u32x4 *)L.p2;
    p.p2k = L.p2k;
    p.c2 = L.c2;
    p.h = L.h;
    p.B = B;
    p.H = L.H;
    p.f = L.f;
    p.theta = L.threshold;
    p.wbits = L.wbits;
    p.ubits = L.ubits;
    p.bundles = (const u32x4 *)L.bundles;
    p.bstride = (size_t)L.nmat * L.cd;
    p.cd = L.cd;
    p.b1 = L.b1;
    p.x = x;
    p.d = L.d;
    p.out = fc1_out(L);
    p.dn_off = (L.nmat - 1) * L.cd;
    p.part1 = L.part1;
    return p;
}

hipError_t launch_score(const LayerView &L, const float *x, int B, bool fc1, const Trace *tr,
                        hipStream_t s) {
    const ScoreParams p = score_params(L, x, B);
    const int cpl2 = pow2_at_least((L.ch + 63) / 64);
    const dim3 grid(L.nq), blk(kThreads);
    if (B == 1) {
        const int k = fc1 ? ASF_K_SCORE_FC1 : ASF_K_SCORE;
        const int cpl1 = fc1_cpl(L.cd);
        // the hottest rows are loaded before scoring when they fit (at most
        // 8 chunks per lane of up and gate rows) and one workgroup per CU
        // covers every owner
        const bool spec = L.nq <= 256;
#define ASF_S1F(WT, G, C1)                                                                 \
    if (spec && C1 * (G ? 2 : 1) <= 8)                                                     \
        ASF_LAUNCH(k, (k_score1<WT, true, G, C1, (C1 * (G ? 2 : 1) <= 8)>), grid, blk, p); \
    else ASF_LAUNCH(k, (k_score1<WT, true, G, C1, false>), grid, blk, p);
#define ASF_S1G(WT, C1) \
    if (L.gated) { ASF_S1F(WT, true, C1) } else { ASF_S1F(WT, false, C1) }
#define ASF_S1W(WT)                                                         \
    if (!fc1) {                                                             \
        ASF_LAUNCH(k, (k_score1<WT, false, false, 1, false>), grid, blk, p); \
    } else switch (cpl1) {                                                  \
    case 1: ASF_S1G(WT, 1) break;                                           \
    case 2: ASF_S1G(WT, 2) break;                                           \
    case 4: ASF_S1G(WT, 4) break;                                           \
    case 8: ASF_S1G(WT, 8) break;                                           \
    case 10: ASF_S1G(WT, 10) break;                                         \
    case 12: ASF_S1G(WT, 12) break;                                         \
    case 14: ASF_S1G(WT, 14) break;                                         \
    default: ASF_S1G(WT, 16) break;                                         \
    }
        if (L.wtype == ASF_F16) { ASF_S1W(1) } else { ASF_S1W(0) }
#undef ASF_S1W
#undef ASF_S1G
#undef ASF_S1F
        return hipGetLastError();
    }
    // batched: score only, then FC1 of the union
    if (L.wtype == ASF_F16) {
        const hipError_t e = launch_score_mm(L, B, tr, s);
        if (e != hipSuccess || !fc1) return e;
        return launch_fc1_mm(L, x, B, 0, nullptr, nullptr, true, tr, s);
    }
#define ASF_S(WT, C2) ASF_LAUNCH(ASF_K_SCORE, (k_score<WT, C2, 4, false, false, 1>), grid, blk, p);
#define ASF_SW(WT)                  \
    switch (cpl2) {                 \
    case 1: ASF_S(WT, 1) break;     \
    case 2: ASF_S(WT, 2) break;     \
    default: ASF_S(WT, 4) break;    \
    }
    ASF_SW(0)   // fp32 weights (fp16 batches went to the matrix cores above)
#undef ASF_SW
#undef ASF_S
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !fc1) return e;
    return launch_fc1(L, x, B, 0, nullptr, nullptr, tr, s);
}

// parameters of the one-launch step: the owner kernels' plus predictor layer
// 1 (rows per owner, waves per row) and the exchange
static ScoreParams step1_params(const LayerView &L, const float *x) {
    ScoreParams p = score_params(L, x, 1);
    p.p1 = L.p1;
    p.c1 = L.c1;
    p.l1_rows = (L.H + L.nq - 1) / L.nq;
    p.l1_wpr = pred1_wpr(L);
    p.xch = L.xch;
    p.xstride = L.xstride;
    p.epoch = L.epoch;
    p.flags = L.dbg;
    return p;
}

// the k_step1 instantiation for layer L (fn) and whether it applies at all
template <int WT, bool G, int C1>
static const void *step1_fn_g(bool spec) {
    if constexpr (C1 * (G ? 2 : 1) <= 8)
        if (spec) return (const void *)k_step1<WT, G, C1, true>;
    return (const void *)k_step1<WT, G, C1, false>;
}

template <int WT, bool G>
static const void *step1_fn_c(int cpl1, bool spec) {
    switch (cpl1) {
    case 1: return step1_fn_g<WT, G, 1>(spec);
    case 2: return step1_fn_g<WT, G, 2>(spec);
    case 4: return step1_fn_g<WT, G, 4>(spec);
    case 8: return step1_fn_g<WT, G, 8>(spec);
    case 10: return step1_fn_g<WT, G, 10>(spec);
    case 12: return step1_fn_g<WT, G, 12>(spec);
    case 14: return step1_fn_g<WT, G, 14>(spec);
    default: return step1_fn_g<WT, G, 16>(spec);
    }
}

static const void *step1_fn(const LayerView &L) {
    const int cpl1 = fc1_cpl(L.cd);
    const bool spec = L.nq <= 256 && cpl1 * (L.gated ? 2 : 1) <= 8;
    if (L.wtype == ASF_F16)
        return L.gated ? step1_fn_c<1, true>(cpl1, spec) : step1_fn_c<1, false>(cpl1, spec);
    return L.gated ? step1_fn_c<0, true>(cpl1, spec) : step1_fn_c<0, false>(cpl1, spec);
}

bool step1_fits(const LayerView &L) {
    // predictor layer 1 in at most two passes of 8 / WPR rows per owner
    const int rows = (L.H + L.nq - 1) / L.nq, rpw = kWaves / pred1_wpr(L);
    if (rows > 2 * rpw || L.H > kMaxHLds || L.cd > kThreads * 4) return false;
    const void *fn = step1_fn(L);
    if (!fn) return false;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, 0) != hipSuccess)
        return false;
    return per_cu >= 1 && (long long)per_cu * L.ncu >= L.nq;
}

hipError_t launch_step1(const LayerView &L, const float *x, const Trace *tr, hipStream_t s) {
    const ScoreParams p = step1_params(L, x);
    const void *fn = step1_fn(L);
    if (!fn) return hipErrorInvalidValue;
    const dim3 grid(L.nq), blk(kThreads);
    void *args[] = {(void *)&p};
    return hipExtLaunchKernel(fn, grid, blk, args, 0, s, ev_start(tr, ASF_K_SCORE_FC1),
                              ev_stop(tr, ASF_K_SCORE_FC1), 0);
}

hipError_t launch_fc1(const LayerView &L, const float *x, int B, int mode, const int32_t *ids,
                      const int32_t *n_ids, const Trace *tr, hipStream_t s) {
    Fc1Params p;
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
    p.out = fc1_out(L);
    const dim3 grid(L.nq), blk(kThreads);
    if (B == 1) {
        const int cpl1 = fc1_cpl(L.cd);
#define ASF_F1(WT, C1)                                                            \
    if (L.gated) ASF_LAUNCH(ASF_K_FC1, (k_fc1_1<WT, true, C1>), grid, blk, p); \
    else ASF_LAUNCH(ASF_K_FC1, (k_fc1_1<WT, false, C1>), grid, blk, p);
#define ASF_F1W(WT)                  \
    switch (cpl1) {                  \
    case 1: ASF_F1(WT, 1) break;     \
    case 2: ASF_F1(WT, 2) break;     \
    case 4: ASF_F1(WT, 4) break;     \
    case 8: ASF_F1(WT, 8) break;     \
    case 10: ASF_F1(WT, 10) break;   \
    case 12: ASF_F1(WT, 12) break;   \
    case 14: ASF_F1(WT, 14) break;   \
    default: ASF_F1(WT, 16) break;   \
    }
        if (L.wtype == ASF_F16) { ASF_F1W(1) } else { ASF_F1W(0) }
#undef ASF_F1W
#undef ASF_F1
        return hipGetLastError();
    }
    if (L.wtype == ASF_F16) return launch_fc1_mm(L, x, B, mode, ids, n_ids, false, tr, s);
    const int cpl1 = pow2_at_least((L.cd + 63) / 64);
#define ASF_F(WT, C1)                                                             \
    if (L.gated) ASF_LAUNCH(ASF_K_FC1, (k_fc1<WT, true, C1>), grid, blk, p); \
    else ASF_LAUNCH(ASF_K_FC1, (k_fc1<WT, false, C1>), grid, blk, p);
#define ASF_FW(WT)                   \
    switch (cpl1) {                  \
    case 1: ASF_F(WT, 1) break;      \
    case 2: ASF_F(WT, 2) break;      \
    case 4: ASF_F(WT, 4) break;      \
    case 8: ASF_F(WT, 8) break;      \
    default: ASF_F(WT, 16) break;    \
    }
    ASF_FW(0)   // fp32 weights (fp16 batches went to the matrix cores above)
#undef ASF_FW
#undef ASF_F
    return hipGetLastError();
}

hipError_t launch_fc2_sum(const LayerView &L, const float *resid, float *y, const Trace *tr,
                          hipStream_t s, bool advance_epoch) {
    const dim3 grid(L.d / 16), blk(kThreads);
    const Fc2SumArgs a{L.part1, L.nq, L.b2, resid, y, advance_epoch ? L.epoch : nullptr};
    const int sq = pow2_at_least((L.nq + kThreads / 4 - 1) / (kThreads / 4));
    switch (sq) {
    case 1: ASF_LAUNCH(ASF_K_FC2, k_fc2_sum<1>, grid, blk, a); break;
    case 2: ASF_LAUNCH(ASF_K_FC2, k_fc2_sum<2>, grid, blk, a); break;
    case 4: ASF_LAUNCH(ASF_K_FC2, k_fc2_sum<4>, grid, blk, a); break;
    default: ASF_LAUNCH(ASF_K_FC2, k_fc2_sum<kSumQ>, grid, blk, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_ffn1(const LayerView &L, const float *x, const int32_t *ids,
                       const int32_t *n_ids, const Trace *tr, hipStream_t s) {
    ScoreParams p = score_params(L, x, 1);
    p.ids = ids;
    p.n_ids = n_ids;
    p.inv = L.inv;
    const bool list = ids != nullptr;
    const dim3 grid(L.nq), blk(kThreads);
    const int cpl1 = fc1_cpl(L.cd);
#define ASF_FFL(WT, G, C1)                                                        \
    if (list) ASF_LAUNCH(ASF_K_FC1, (k_ffn1<WT, G, C1, true>), grid, blk, p);  \
    else ASF_LAUNCH(ASF_K_FC1, (k_ffn1<WT, G, C1, false>), grid, blk, p);
#define ASF_FF(WT, C1) \
    if (L.gated) { ASF_FFL(WT, true, C1) } else { ASF_FFL(WT, false, C1) }
#define ASF_FFW(WT)                  \
    switch (cpl1) {                  \
    case 1: ASF_FF(WT, 1) break;     \
    case 2: ASF_FF(WT, 2) break;     \
    case 4: ASF_FF(WT, 4) break;     \
    case 8: ASF_FF(WT, 8) break;     \
    case 10: ASF_FF(WT, 10) break;   \
    case 12: ASF_FF(WT, 12) break;   \
    case 14: ASF_FF(WT, 14) break;   \
    default: ASF_FF(WT, 16) break;   \
    }
    if (L.wtype == ASF_F16) { ASF_FFW(1) } else { ASF_FFW(0) }
#undef ASF_FFW
#undef ASF_FF
#undef ASF_FFL
    return hipGetLastError();
}

hipError_t launch_ffn1_pred1(const LayerView &L, const LayerView *N, const float *x,
                             const Trace *tr, hipStream_t s) {
    if (!N || N->wtype != L.wtype) {
        const hipError_t e = launch_ffn1(L, x, nullptr, nullptr, tr, s);
        if (e != hipSuccess || !N) return e;
        return launch_pred_l1(*N, x, 1, nullptr, s);
    }
    const ScoreParams p = score_params(L, x, 1);
    const Pred1Args a = pred1_args(*N, x);
    const dim3 grid(L.nq + pred1_blocks(*N)), blk(kThreads);
    const int cpl1 = fc1_cpl(L.cd);
#define ASF_FP(WT, C1)                                                                        \
    if (L.gated) ASF_LAUNCH(ASF_K_FC1, (k_ffn1_pred1<WT, true, C1>), grid, blk, p, L.nq, a);  \
    else ASF_LAUNCH(ASF_K_FC1, (k_ffn1_pred1<WT, false, C1>), grid, blk, p, L.nq, a);
#define ASF_FPW(WT)                  \
    switch (cpl1) {                  \
    case 1: ASF_FP(WT, 1) break;     \
    case 2: ASF_FP(WT, 2) break;     \
    case 4: ASF_FP(WT, 4) break;     \
    case 8: ASF_FP(WT, 8) break;     \
    case 10: ASF_FP(WT, 10) break;   \
    case 12: ASF_FP(WT, 12) break;   \
    case 14: ASF_FP(WT, 14) break;   \
    default: ASF_FP(WT, 16) break;   \
    }
    if (L.wtype == ASF_F16) { ASF_FPW(1) } else { ASF_FPW(0) }
#undef ASF_FPW
#undef ASF_FP
    return hipGetLastError();
}

hipError_t launch_score1_fc2sum(const LayerView *N, const LayerView &L, const float *resid,
                                float *y, const Trace *tr, hipStream_t s) {
    if (!N) return launch_fc2_sum(L, resid, y, tr, s);
    const ScoreParams p = score_params(*N, nullptr, 1);
    const Fc2SumArgs a{L.part1, L.nq, L.b2, resid, y, nullptr};
    const dim3 grid(N->nq + L.d / 16), blk(kThreads);
    const int sq = pow2_at_least((L.nq + kThreads / 4 - 1) / (kThreads / 4));
#define ASF_SF(WT)                                                                              \
    switch (sq) {                                                                               \
    case 1: ASF_LAUNCH(ASF_K_FC2, (k_score1_fc2sum<WT, 1>), grid, blk, p, N->nq, a); break;     \
    case 2: ASF_LAUNCH(ASF_K_FC2, (k_score1_fc2sum<WT, 2>), grid, blk, p, N->nq, a); break;     \
    case 4: ASF_LAUNCH(ASF_K_FC2, (k_score1_fc2sum<WT, 4>), grid, blk, p, N->nq, a); break;     \
    default: ASF_LAUNCH(ASF_K_FC2, (k_score1_fc2sum<WT, kSumQ>), grid, blk, p, N->nq, a); break; \
    }
    if (N->wtype == ASF_F16) { ASF_SF(1) } else { ASF_SF(0) }
#undef ASF_SF
    return hipGetLastError();
}

hipError_t launch_exact1(const LayerView &L, const float *x, bool mask_only, const Trace *tr,
                         hipStream_t s) {
    ScoreParams p = score_params(L, x, 1);
    if (mask_only) p.part1 = nullptr;
    const dim3 grid(L.nq), blk(kThreads);
    const int cpl1 = fc1_cpl(L.cd);
#define ASF_EX(WT, C1)                                                              \
    if (L.gated) ASF_LAUNCH(ASF_K_FC1, (k_exact1<WT, true, C1>), grid, blk, p);  \
    else ASF_LAUNCH(ASF_K_FC1, (k_exact1<WT, false, C1>), grid, blk, p);
#define ASF_EXW(WT)                  \
    switch (cpl1) {                  \
    case 1: ASF_EX(WT, 1) break;     \
    case 2: ASF_EX(WT, 2) break;     \
    case 4: ASF_EX(WT, 4) break;     \
    case 8: ASF_EX(WT, 8) break;     \
    case 10: ASF_EX(WT, 10) break;   \
    case 12: ASF_EX(WT, 12) break;   \
    case 14: ASF_EX(WT, 14) break;   \
    default: ASF_EX(WT, 16) break;   \
    }
    if (L.wtype == ASF_F16) { ASF_EXW(1) } else { ASF_EXW(0) }
#undef ASF_EXW
#undef ASF_EX
    return hipGetLastError();
}

hipError_t launch_count_bits(const LayerView &L, uint32_t *counts, hipStream_t s) {
    hipLaunchKernelGGL(k_count_bits, dim3((L.f + 255) / 256), dim3(256), 0, s,
                       (const uint64_t *)L.wbits, L.f, L.nq, (const int32_t *)L.perm, counts);
    return hipGetLastError();
}

hipError_t launch_rank_table(const uint32_t *counts, int f, int32_t *table, hipStream_t s) {
    hipLaunchKernelGGL(k_rank_table, dim3((f + kRankTile - 1) / kRankTile), dim3(kRankTile), 0, s,
                       counts, f, table);
    return hipGetLastError();
}

hipError_t launch_fc2(const LayerView &L, int B, bool listed, const float *resid, float *y,
                      const Trace *tr, hipStream_t s, bool all_rows) {
    Fc2Params p;
    p.bundles = (const u32x4 *)L.bundles;
    p.bstride = (size_t)L.nmat * L.cd;
    p.dn_off = (L.nmat - 1) * L.cd;
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
    if (B > 1 && L.wtype == ASF_F16) return launch_fc2_mm(L, B, all_rows, resid, y, tr, s);
    const dim3 grid(kSlices * kGroups), blk(kThreads);
    if (L.wtype == ASF_F16) {
        ASF_LAUNCH(ASF_K_FC2, (k_fc2<1, 1>), grid, blk, p);   // one token (batches: above)
    } else {
        if (B == 1) ASF_LAUNCH(ASF_K_FC2, (k_fc2<0, 1>), grid, blk, p);
        else ASF_LAUNCH(ASF_K_FC2, (k_fc2<0, 4>), grid, blk, p);
    }
    return hipGetLastError();
}

hipError_t launch_head_predict(const HeadView &V, const float *x, int B, uint64_t *masks,
                               int32_t *heads, int32_t *count, hipStream_t s) {
    // layer 1 through the FFN predictor's launcher on a view of the head
    // predictor's rows and scratch: one token as a GEMV, 2-4 fp16 tokens with
    // the weights held while the tokens go by, more on the matrix cores
    LayerView lv = {};
    lv.d = V.d;
    lv.H = V.H;
    lv.f = V.nh;
    lv.max_batch = V.max_batch;
    lv.wtype = V.wtype;
    lv.ws = V.ws;
    lv.cd = V.cd;
    lv.ch = V.ch;
    lv.p1 = V.q1;
    lv.c1 = V.c1;
    lv.h = V.h;
    lv.h16 = V.h16;
    lv.x16 = V.x16;
    lv.pred_part = V.pred_part;
    lv.ncu = V.ncu;
    if (launch_pred_l1(lv, x, B, nullptr, s) != hipSuccess) return hipGetLastError();
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // layer 2, threshold, masks (and lists of a single word per token)
    const HeadArgs a{(const u32x4 *)V.q2, V.c2, V.h, V.H, V.nh, V.words, V.threshold,
                     V.wbits, masks, heads, count};
    const dim3 grid(V.words, B), blk(kThreads);
    const int cpl2 = pow2_at_least((V.ch + 63) / 64);
    if (V.wtype == ASF_F16) {
        if (cpl2 == 1) hipLaunchKernelGGL((k_head_score<1, 1>), grid, blk, 0, s, a);
        else if (cpl2 == 2) hipLaunchKernelGGL((k_head_score<1, 2>), grid, blk, 0, s, a);
        else hipLaunchKernelGGL((k_head_score<1, 4>), grid, blk, 0, s, a);
    } else {
        if (cpl2 == 1) hipLaunchKernelGGL((k_head_score<0, 1>), grid, blk, 0, s, a);
        else if (cpl2 == 2) hipLaunchKernelGGL((k_head_score<0, 2>), grid, blk, 0, s, a);
        else hipLaunchKernelGGL((k_head_score<0, 4>), grid, blk, 0, s, a);
    }
    e = hipGetLastError();
    if (e != hipSuccess || V.words == 1 || (!heads && !count)) return e;
    hipLaunchKernelGGL(k_head_list, dim3(B), dim3(64), 0, s, (const uint64_t *)V.wbits, V.words,
                       V.nh, heads, count);
    return hipGetLastError();
}

hipError_t launch_check_ids(const int32_t *ids, const int32_t *n_ids, int n_fixed, int f,
                            uint32_t *bitmap, unsigned *flags, hipStream_t s) {
    const int words = (f + 31) / 32;
    hipLaunchKernelGGL(k_zero_u32, dim3((words + 255) / 256), dim3(256), 0, s, bitmap, words);
    hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(64), 0, s, (uint32_t *)flags, 1);
    hipLaunchKernelGGL(k_check_ids, dim3((f + 255) / 256), dim3(256), 0, s, ids, n_ids, n_fixed, f,
                       bitmap, flags);
    return hipGetLastError();
}

static ListArgs list_args(const LayerView &L, int B, int32_t *active_ids, int32_t *n_active,
                          uint64_t *token_masks) {
    return ListArgs{(const uint64_t *)L.ubits, (const uint64_t *)L.wbits, B, L.f, L.nq, L.words,
                    (const int32_t *)L.perm, token_masks, L.slots, L.count, active_ids, n_active};
}

hipError_t launch_list(const LayerView &L, int B, int32_t *active_ids, int32_t *n_active,
                       uint64_t *token_masks, const Trace *tr, hipStream_t s) {
    const dim3 grid((L.f + kListSlots - 1) / kListSlots), blk(kThreads);
    const ListArgs a = list_args(L, B, active_ids, n_active, token_masks);
    if (token_masks) ASF_LAUNCH(ASF_K_LIST, k_list<true>, grid, blk, a);
    else ASF_LAUNCH(ASF_K_LIST, k_list<false>, grid, blk, a);
    return hipGetLastError();
}

hipError_t launch_fc2_sum_list(const LayerView &L, const float *resid, float *y,
                               int32_t *active_ids, int32_t *n_active, const Trace *tr,
                               hipStream_t s, bool advance_epoch) {
    const int nsum = L.d / 16, nlist = (L.f + kListSlots - 1) / kListSlots;
    const dim3 grid(nsum + nlist), blk(kThreads);
    const Fc2SumArgs a{L.part1, L.nq, L.b2, resid, y, advance_epoch ? L.epoch : nullptr};
    const ListArgs l = list_args(L, 1, active_ids, n_active, nullptr);
    const int sq = pow2_at_least((L.nq + kThreads / 4 - 1) / (kThreads / 4));
    switch (sq) {
    case 1: ASF_LAUNCH(ASF_K_FC2, k_fc2_sum_list<1>, grid, blk, a, nsum, l); break;
    case 2: ASF_LAUNCH(ASF_K_FC2, k_fc2_sum_list<2>, grid, blk, a, nsum, l); break;
    case 4: ASF_LAUNCH(ASF_K_FC2, k_fc2_sum_list<4>, grid, blk, a, nsum, l); break;
    default: ASF_LAUNCH(ASF_K_FC2, k_fc2_sum_list<kSumQ>, grid, blk, a, nsum, l); break;
    }
    return hipGetLastError();
}

}  // namespace asf
