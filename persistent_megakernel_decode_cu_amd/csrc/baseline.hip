// One-kernel-per-op HIP baseline of the same decode step, for comparison with
// the megakernel: every operator is its own launch and every launch boundary is
// a device-wide barrier, the execution model the pages contrast the megakernel
// with (Hazy Research megakernel news page, section 3, "problems of existing
// methods": hundreds of short kernels, launch cost, idle SMs in the tail of
// each kernel, waiting for weights after each launch; cloud.baidu.com
// explainer, section 3: per-operator kernels write their intermediates to
// memory).  Same arithmetic as the megakernel (bf16 weights, fp32 activations
// and accumulation), independent code.
//
// One sequence: vector-ALU GEMVs with fused epilogues.  Several sequences: the
// projections run on the matrix cores, each in slices of K whose partial sums the
// next kernel adds as it reads them (RoPE adds the Q/K/V slices, RMSNorm the
// O-projection and down-projection slices together with the residual, the SiLU
// kernel the gate/up slices), and every projection input is stored once as two
// bf16 parts (hi + lo) in operand-ready rows.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "../../include/mk.h"

namespace mkb {

__device__ __forceinline__ float bflo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bfhi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float warp_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float warp_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
// v as two bf16 parts: hi = v rounded, lo = the remainder rounded (hi + lo within 2^-16 |v|)
__device__ __forceinline__ void store_split(uint16_t* xs, size_t plane, size_t i, float v) {
    const uint16_t hi = to_bf16(v);
    xs[i] = hi;
    xs[plane + i] = to_bf16(v - bf(hi));
}

// x[b] = embedding row of token b; grid (blocks, B)
__global__ void k_embed(const uint16_t* E, const int32_t* tok, float* x, int h) {
    const uint16_t* row = E + (size_t)tok[blockIdx.y] * h;
    float* xb = x + (size_t)blockIdx.y * h;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < h; i += gridDim.x * blockDim.x) xb[i] = bf(row[i]);
}

// One workgroup of 1024 threads per sequence b.  The residual first:
// xout[b] = xin[b] + sum over the ks slices of part[slice][b] (ks = 0: xout = xin,
// not written), then n = xout * g / sqrt(mean(xout^2) + eps), stored as fp32 into xn
// (if not null) and as two bf16 parts into xs[2][B][h] (if not null).
__global__ void __launch_bounds__(1024) k_rmsnorm(const float* xin, const float* __restrict__ part, int ks, float* xout,
                                                  const uint16_t* g, float eps, float* xn, uint16_t* xs, int h) {
    __shared__ float red[16];
    const int b = blockIdx.x, B = gridDim.x;
    const float* xi = xin + (size_t)b * h;
    float* xo = xout + (size_t)b * h;
    float ss = 0.f;
    for (int i = threadIdx.x; i < h; i += 1024) {
        float v = xi[i];
#pragma unroll 8
        for (int s = 0; s < ks; ++s) v += part[((size_t)s * B + b) * h + i];
        if (ks) xo[i] = v;
        ss += v * v;
    }
    ss = warp_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < 16; ++w) tot += red[w];
    const float r = 1.0f / sqrtf(tot / (float)h + eps);
    const float* xr = ks ? xo : xi;  // each thread reads back only what it wrote
    for (int i = threadIdx.x; i < h; i += 1024) {
        const float v = xr[i] * r * bf(g[i]);
        if (xn) xn[(size_t)b * h + i] = v;
        if (xs) store_split(xs, (size_t)B * h, (size_t)b * h + i, v);
    }
}

// One sequence: y[r] = W[r,:] . x (+ epilogue): each wave computes R consecutive rows,
// each lane 8 columns per 512-column stride; K is a multiple of 512.
enum Epi { EPI_STORE = 0, EPI_RESID = 1, EPI_SILU_MUL = 2 };
template <int K, int R, int EPI>
__global__ void __launch_bounds__(256) k_gemv(const uint16_t* __restrict__ W, const float* __restrict__ x,
                                              float* __restrict__ y, int rows, const float* __restrict__ aux,
                                              const uint16_t* __restrict__ W2) {
    const int lane = threadIdx.x & 63;
    const int r0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
    if (r0 >= rows) return;
    float xv[K / 64];
#pragma unroll
    for (int j = 0; j < K / 512; ++j) {
        const float4 a = *(const float4*)(x + j * 512 + lane * 8);
        const float4 b = *(const float4*)(x + j * 512 + lane * 8 + 4);
        xv[j * 8 + 0] = a.x; xv[j * 8 + 1] = a.y; xv[j * 8 + 2] = a.z; xv[j * 8 + 3] = a.w;
        xv[j * 8 + 4] = b.x; xv[j * 8 + 5] = b.y; xv[j * 8 + 6] = b.z; xv[j * 8 + 7] = b.w;
    }
    constexpr int NM = EPI == EPI_SILU_MUL ? 2 : 1;
    float acc[NM][R];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const uint16_t* Wm = m == 0 ? W : W2;
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            const int r = min(r0 + rr, rows - 1);
            const uint4* row = (const uint4*)(Wm + (size_t)r * K);
            uint4 w[K / 512];
#pragma unroll
            for (int j = 0; j < K / 512; ++j) w[j] = row[j * 64 + lane];
            float a = 0.f;
#pragma unroll
            for (int j = 0; j < K / 512; ++j) {
                a = fmaf(bflo(w[j].x), xv[j * 8 + 0], a);
                a = fmaf(bfhi(w[j].x), xv[j * 8 + 1], a);
                a = fmaf(bflo(w[j].y), xv[j * 8 + 2], a);
                a = fmaf(bfhi(w[j].y), xv[j * 8 + 3], a);
                a = fmaf(bflo(w[j].z), xv[j * 8 + 4], a);
                a = fmaf(bfhi(w[j].z), xv[j * 8 + 5], a);
                a = fmaf(bflo(w[j].w), xv[j * 8 + 6], a);
                a = fmaf(bfhi(w[j].w), xv[j * 8 + 7], a);
            }
            acc[m][rr] = a;
        }
    }
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
        const int r = r0 + rr;
        const float v = warp_sum(acc[0][rr]);
        if (EPI == EPI_SILU_MUL) {
            const float u = warp_sum(acc[NM - 1][rr]);
            if (lane == 0 && r < rows) y[r] = v / (1.0f + __expf(-v)) * u;
        } else if (lane == 0 && r < rows) {
            y[r] = EPI == EPI_RESID ? aux[r] + v : v;
        }
    }
}

// Several sequences: part[slice][b][r] = W[r, slice] . X[b, slice] on
// v_mfma_f32_16x16x32_bf16.  The weights are the A operand, read from the caller's
// [rows][K] matrices (lane l: row l % 16, columns 8 (l / 16) .. +7 of each 32-column
// step); the activations are the B operand, read from X = [2][B][K] bf16 (hi parts,
// then lo parts), sequence b in column b % 16 of column group b / 16; one product per
// part, fp32 accumulation.  Up to three matrices stacked as one of R rows (matrix m
// from row rb[m]).  A wave owns RG row groups of 16 rows and one of ks equal slices
// of K, and streams its slice in chunks of U 32-column steps, loading the next chunk
// while it multiplies the current one.
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

struct GemmArgs {
    const uint16_t* W[3];
    int rb[3];  // first stacked row of each matrix (unused ones: R)
    int R, K, ks, B;
    const uint16_t* X;
    float* out;
};

template <int RG, int NG, int U>
struct Chunk {
    u32x4v a[U][RG], h[U][NG], l[U][NG];
};

template <int RG, int NG, int U>
__device__ __forceinline__ void load_chunk(Chunk<RG, NG, U>& c, const uint16_t* wl, size_t K,
                                           const uint16_t* const (&xh)[NG], const uint16_t* const (&xl)[NG], int kk) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
            c.a[u][rg] = __builtin_nontemporal_load((const u32x4v*)(wl + (size_t)rg * 16 * K + kk + 32 * u));
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            c.h[u][g] = *(const u32x4v*)(xh[g] + kk + 32 * u);
            c.l[u][g] = *(const u32x4v*)(xl[g] + kk + 32 * u);
        }
    }
}
template <int RG, int NG, int U>
__device__ __forceinline__ void mul_chunk(const Chunk<RG, NG, U>& c, f32x4v (&acc)[RG][NG]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                acc[rg][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, c.a[u][rg]),
                                                                     __builtin_bit_cast(bf16x8v, c.h[u][g]), acc[rg][g],
                                                                     0, 0, 0);
                acc[rg][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, c.a[u][rg]),
                                                                     __builtin_bit_cast(bf16x8v, c.l[u][g]), acc[rg][g],
                                                                     0, 0, 0);
            }
}

template <int RG, int NG, int U>
__global__ void __launch_bounds__(256) k_gemm_b(GemmArgs p) {
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int tiles = p.R / (16 * RG);
    if (gw >= tiles * p.ks) return;
    const int tile = gw / p.ks, s = gw - tile * p.ks;
    const int r0 = tile * 16 * RG;
    const int m = (r0 >= p.rb[1] ? 1 : 0) + (r0 >= p.rb[2] ? 1 : 0);
    const int KS = p.K / p.ks, k0 = s * KS;
    const int n = lane & 15, q = lane >> 4;
    const size_t K = (size_t)p.K;
    const uint16_t* wl = p.W[m] + (size_t)(r0 - p.rb[m] + n) * K + k0 + 8 * q;
    const uint16_t* xh[NG];
    const uint16_t* xl[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        // columns past the last sequence read a valid row; their results are not stored
        const int b = min(g * 16 + n, p.B - 1);
        xh[g] = p.X + (size_t)b * K + k0 + 8 * q;
        xl[g] = xh[g] + (size_t)p.B * K;
    }
    f32x4v acc[RG][NG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int g = 0; g < NG; ++g) acc[rg][g] = f32x4v{0.f, 0.f, 0.f, 0.f};
    constexpr int CW = 32 * U;  // columns per chunk
    const int nc = KS / CW;
    Chunk<RG, NG, U> c0, c1;
    load_chunk(c0, wl, K, xh, xl, 0);
    for (int c = 0; c < nc; c += 2) {
        if (c + 1 < nc) load_chunk(c1, wl, K, xh, xl, (c + 1) * CW);
        mul_chunk(c0, acc);
        if (c + 1 < nc) {
            if (c + 2 < nc) load_chunk(c0, wl, K, xh, xl, (c + 2) * CW);
            mul_chunk(c1, acc);
        }
    }
    // lane (n, q) holds rows 4 q .. 4 q + 3 of each row group for sequence 16 g + n
#pragma unroll
    for (int g = 0; g < NG; ++g)
        if (g * 16 + n < p.B)
#pragma unroll
            for (int rg = 0; rg < RG; ++rg)
                *(f32x4v*)(p.out + ((size_t)s * p.B + g * 16 + n) * p.R + r0 + rg * 16 + 4 * q) = acc[rg][g];
}

// m[b][r] = SiLU(gate) * up from the ks slices of part[slice][b][0 .. 2 rows) (gate
// rows, then up rows), stored as two bf16 parts into ms[2][B][rows]
__global__ void k_silu_mul(const float* __restrict__ part, int ks, int B, int rows, uint16_t* __restrict__ ms) {
    const int n = B * rows;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
        const int b = i / rows, r = i - b * rows;
        float g = 0.f, u = 0.f;
        for (int s = 0; s < ks; ++s) {
            const float* ps = part + ((size_t)s * B + b) * 2 * rows;
            g += ps[r];
            u += ps[rows + r];
        }
        store_split(ms, (size_t)n, i, g / (1.0f + __expf(-g)) * u);
    }
}

// Sequence blockIdx.y: q, k, v = the sum of the ks slices of src[slice][b][0 .. R3)
// (q at 0, k at nq d, v at (nq + nkv) d; R3 = (nq + 2 nkv) d); RoPE on q (stored into
// qo[b]) and k (pairs j, j + d/2 of each head), and the K/V append (bf16) at slot
// pos[b] of this layer's [B][nkv][C][d] caches
__global__ void k_rope_append(const float* __restrict__ src, int ks, float* __restrict__ qo, const float2* rope,
                              const int32_t* pos, int nq, int nkv, int d, uint16_t* kc, uint16_t* vc, int C) {
    const int b = blockIdx.y, B = gridDim.y;
    const int half = d / 2;
    const int P = pos[b];
    const int R3 = (nq + 2 * nkv) * d;
    const int n = (nq + nkv) * half;
    auto val = [&](int i) {
        float v = 0.f;
        for (int s = 0; s < ks; ++s) v += src[((size_t)s * B + b) * R3 + i];
        return v;
    };
    qo += (size_t)b * nq * d;
    kc += (size_t)b * nkv * C * d;
    vc += (size_t)b * nkv * C * d;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n + nkv * d; i += gridDim.x * blockDim.x) {
        if (i < n) {
            const int hd = i / half, j = i % half;
            const float2 cs = rope[(size_t)P * half + j];
            const float lo = val(hd * d + j), hi = val(hd * d + j + half);
            const float a = lo * cs.x - hi * cs.y, c = lo * cs.y + hi * cs.x;
            if (hd < nq) {
                qo[(size_t)hd * d + j] = a;
                qo[(size_t)hd * d + j + half] = c;
            } else {
                const int g = hd - nq;
                kc[((size_t)g * C + P) * d + j] = to_bf16(a);
                kc[((size_t)g * C + P) * d + j + half] = to_bf16(c);
            }
        } else {
            const int t = i - n, g = t / d, e = t % d;
            vc[((size_t)g * C + P) * d + e] = to_bf16(val((nq + nkv) * d + t));
        }
    }
}

// Attention partial of KV group blockIdx.x over chunk blockIdx.y of sequence blockIdx.z's
// context: one wave per query head of the group (the group's waves read the same K/V
// rows, so they come from HBM once).  Per block of 64 positions, the wave reads the
// K and V rows with lane (row r, dimension group dg) taking 16 bytes (8 dimensions)
// of row j * (64 / (d / 8)) + r for every j, all loads issued first.  Scores: the
// 8-dimension products summed over a row's lanes, then handed to one position per
// lane.  P.V: each lane accumulates its 8 dimensions over its rows, and the rows
// are summed at the end.  Writes (m, l, o[d]) to part[b][head][chunk].
template <int D>
__global__ void __launch_bounds__(512) k_attn_part(const float* q, const uint16_t* kc, const uint16_t* vc,
                                                   const int32_t* pos, int nq, int nkv, int C, int splits,
                                                   float* part) {
    constexpr int LPR = D / 8;     // lanes per row
    constexpr int PPI = 64 / LPR;  // rows per load
    constexpr int NV = 64 / PPI;   // loads per lane per block of 64 positions (of K, and of V)
    const int g = blockIdx.x, c = blockIdx.y, b = blockIdx.z;
    const int grp = nq / nkv, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int hq = g * grp + wave;
    const int dg = lane % LPR, pg = lane / LPR;
    const int n = pos[b] + 1;
    const int lc = (n + splits - 1) / splits;
    const int p0 = min(n, c * lc), p1 = min(n, p0 + lc);
    const uint16_t* K = kc + ((size_t)b * nkv + g) * C * D;
    const uint16_t* V = vc + ((size_t)b * nkv + g) * C * D;
    __shared__ float ws[8][64];
    const float scale = 1.0f / sqrtf((float)D);
    // this lane's 8 query dimensions, pre-scaled
    float qv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[i] = q[((size_t)b * nq + hq) * D + dg * 8 + i] * scale;
    float M = -INFINITY, L = 0.f, ov[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) ov[i] = 0.f;
    for (int b0 = p0; b0 < p1; b0 += 64) {
        const int p = b0 + lane;
        uint4 kw[NV], vv[NV];
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const size_t row = (size_t)min(b0 + j * PPI + pg, p1 - 1) * D + dg * 8;
            kw[j] = *(const uint4*)(K + row);
            vv[j] = *(const uint4*)(V + row);
        }
        float sc[NV];
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            float t = bflo(kw[j].x) * qv[0] + bfhi(kw[j].x) * qv[1] + bflo(kw[j].y) * qv[2] + bfhi(kw[j].y) * qv[3] +
                      bflo(kw[j].z) * qv[4] + bfhi(kw[j].z) * qv[5] + bflo(kw[j].w) * qv[6] + bfhi(kw[j].w) * qv[7];
#pragma unroll
            for (int o = 1; o < LPR; o <<= 1) t += __shfl_xor(t, o, 64);
            sc[j] = t;
        }
        // position b0 + lane: row lane % PPI of load lane / PPI
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const float t = __shfl(sc[j], (lane % PPI) * LPR, 64);
            if (lane / PPI == j) a = t;
        }
        const float s = p < p1 ? a : -INFINITY;
        const float mn = fmaxf(M, warp_max(s));
        const float corr = __expf(M - mn);
        const float e = p < p1 ? __expf(s - mn) : 0.f;
        L = L * corr + warp_sum(e);
        M = mn;
        ws[wave][lane] = e;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; ++i) ov[i] *= corr;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const float wgt = ws[wave][j * PPI + pg];  // 0 past the chunk's end
            ov[0] = fmaf(wgt, bflo(vv[j].x), ov[0]);
            ov[1] = fmaf(wgt, bfhi(vv[j].x), ov[1]);
            ov[2] = fmaf(wgt, bflo(vv[j].y), ov[2]);
            ov[3] = fmaf(wgt, bfhi(vv[j].y), ov[3]);
            ov[4] = fmaf(wgt, bflo(vv[j].z), ov[4]);
            ov[5] = fmaf(wgt, bfhi(vv[j].z), ov[5]);
            ov[6] = fmaf(wgt, bflo(vv[j].w), ov[6]);
            ov[7] = fmaf(wgt, bfhi(vv[j].w), ov[7]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i) ov[i] += __shfl_xor(ov[i], off, 64);
    float* dst = part + (((size_t)b * nq + hq) * splits + c) * (D + 2);
    if (lane == 0) {
        dst[0] = M;
        dst[1] = L;
    }
    if (pg == 0)
#pragma unroll
        for (int i = 0; i < 8; ++i) dst[2 + dg * 8 + i] = ov[i];
}

// Merge of the chunk partials (splits <= 64) of query head blockIdx.x of sequence
// blockIdx.y, 64 threads: one chunk per lane for the maximum and the denominator, one
// dimension per lane for the weighted sum.  Output as fp32 a[b][head][t] (if not
// null) and as two bf16 parts into as[2][B][nq d] (if not null).
__global__ void __launch_bounds__(64) k_attn_merge(const float* part, int nq, int splits, int D, float* a,
                                                   uint16_t* as) {
    __shared__ float sc[64];
    const int hq = blockIdx.x, b = blockIdx.y, B = gridDim.y, lane = threadIdx.x;
    const float* src = part + ((size_t)b * nq + hq) * splits * (D + 2);
    const float m = lane < splits ? src[lane * (D + 2)] : -INFINITY;
    const float Mx = warp_max(m);
    const float w = m == -INFINITY ? 0.f : __expf(m - Mx);
    const float den = warp_sum(lane < splits ? w * src[lane * (D + 2) + 1] : 0.f);
    sc[lane] = w;
    __syncthreads();
    for (int t = lane; t < D; t += 64) {
        float num = 0.f;
#pragma unroll 8
        for (int c = 0; c < splits; ++c) num = fmaf(sc[c], src[c * (D + 2) + 2 + t], num);
        const size_t i = ((size_t)b * nq + hq) * D + t;
        if (a) a[i] = num / den;
        if (as) store_split(as, (size_t)B * nq * D, i, num / den);
    }
}

// (value, index) of the larger of two candidates; equal values: the lower index
__device__ __forceinline__ void better(float& bv, int& bi, float ov, int oi) {
    if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
    }
}

// argmax over the logits of sequence blockIdx.y: stage 1 per block (value, lowest
// index) over a grid-stride share, stage 2 over the blocks
__global__ void __launch_bounds__(256) k_argmax1(const float* v, int n, float* bv, int* bi) {
    __shared__ float sv[256];
    __shared__ int si[256];
    v += (size_t)blockIdx.y * n;
    float best = -INFINITY;
    int idx = 0x7fffffff;
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256)
        if (v[i] > best) {
            best = v[i];
            idx = i;
        }
    sv[threadIdx.x] = best;
    si[threadIdx.x] = idx;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) better(sv[threadIdx.x], si[threadIdx.x], sv[threadIdx.x + s], si[threadIdx.x + s]);
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        bv[blockIdx.y * gridDim.x + blockIdx.x] = sv[0];
        bi[blockIdx.y * gridDim.x + blockIdx.x] = si[0];
    }
}
// one workgroup of 256 threads per sequence; nb <= 256
__global__ void __launch_bounds__(256) k_argmax2(const float* bv, const int* bi, int nb, int* next, const float* x,
                                                 float* hidden, int h, int32_t* tok_out, int32_t* pos_inout) {
    __shared__ float sv[256];
    __shared__ int si[256];
    const int b = blockIdx.x, t = threadIdx.x;
    sv[t] = t < nb ? bv[b * nb + t] : -INFINITY;
    si[t] = t < nb ? bi[b * nb + t] : 0x7fffffff;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (t < s) better(sv[t], si[t], sv[t + s], si[t + s]);
        __syncthreads();
    }
    if (t == 0) {
        next[b] = si[0];
        if (tok_out) tok_out[b] = si[0];
        if (pos_inout) pos_inout[b] += 1;
    }
    for (int i = t; i < h; i += 256) hidden[(size_t)b * h + i] = x[(size_t)b * h + i];
}

}  // namespace mkb

using namespace mkb;

struct mkb_handle {
    mk_model_desc desc;
    std::vector<mk_layer_weights> layers;
    int B = 1, C = 0, S = 8, nb_arg = 256;
    int launches = 0;      // kernels enqueued by the last step
    float* buf = nullptr;  // activations, partials and argmax scratch
    float *x, *xn, *xb, *qkv, *q, *a, *m, *lg, *part, *gpart, *bv, *hidden;
    uint16_t *xs, *as, *ms;  // projection inputs as two bf16 parts (several sequences)
    int *bi, *next;
    float2* rope = nullptr;
};

namespace {

template <int K, int EPI>
void gemv(const uint16_t* W, const float* x, float* y, int rows, const float* aux, const uint16_t* W2, hipStream_t s) {
    constexpr int R = 2;
    const int blocks = (rows + 4 * R - 1) / (4 * R);
    hipLaunchKernelGGL((k_gemv<K, R, EPI>), dim3(blocks), dim3(256), 0, s, W, x, y, rows, aux, W2);
}
template <int EPI>
void gemv_k(int K, const uint16_t* W, const float* x, float* y, int rows, const float* aux, const uint16_t* W2,
            hipStream_t s) {
    switch (K) {
        case 512: gemv<512, EPI>(W, x, y, rows, aux, W2, s); break;
        case 1024: gemv<1024, EPI>(W, x, y, rows, aux, W2, s); break;
        case 2048: gemv<2048, EPI>(W, x, y, rows, aux, W2, s); break;
        case 4096: gemv<4096, EPI>(W, x, y, rows, aux, W2, s); break;
        default: gemv<8192, EPI>(W, x, y, rows, aux, W2, s); break;  // K checked at create
    }
}

// Work split of one several-sequence projection of R stacked rows over K columns:
// RG row groups of 16 per wave (4 for the large matrices), and K cut into ks
// slices of at least 256 columns until there are about 1024 waves (ks = 1 when
// the result must be whole, as for the logits).
struct GemmPlan {
    int RG, ks, waves;
};
GemmPlan plan_gemm(int R, int K, bool whole) {
    GemmPlan p;
    p.RG = (R >= 8192 && R % 64 == 0) ? 4 : 1;
    const int tiles = R / (16 * p.RG);
    p.ks = 1;
    while (!whole && tiles * p.ks < 1024 && K % (512 * p.ks) == 0) p.ks *= 2;
    p.waves = tiles * p.ks;
    return p;
}

}  // namespace

// Several sequences: out[slice][b][r] for the stacked matrices W[0..nmat) of rows
// rows[0..nmat); returns the number of K slices written.
static int project_b(mkb_handle* hb, const uint16_t* const* W, const int* rows, int nmat, int K, const uint16_t* X,
                     float* out, bool whole, hipStream_t s) {
    GemmArgs a;
    int R = 0;
    for (int i = 0; i < 3; ++i) {
        a.W[i] = i < nmat ? W[i] : W[0];
        a.rb[i] = R;
        if (i < nmat) R += rows[i];
    }
    for (int i = nmat; i < 3; ++i) a.rb[i] = R;
    const GemmPlan p = plan_gemm(R, K, whole);
    a.R = R;
    a.K = K;
    a.ks = p.ks;
    a.B = hb->B;
    a.X = X;
    a.out = out;
    const dim3 grid((p.waves + 3) / 4), blk(256);
    // column groups of 16 sequences per wave: 1, 2 or 4 (33..64 sequences; a third group's
    // columns past the last sequence read a valid row and are not stored)
    const int ng = hb->B > 32 ? 4 : hb->B > 16 ? 2 : 1;
    if (p.RG == 4) {
        if (ng == 4) hipLaunchKernelGGL((k_gemm_b<4, 4, 1>), grid, blk, 0, s, a);
        else if (ng == 2) hipLaunchKernelGGL((k_gemm_b<4, 2, 2>), grid, blk, 0, s, a);
        else hipLaunchKernelGGL((k_gemm_b<4, 1, 4>), grid, blk, 0, s, a);
    } else {
        if (ng == 4) hipLaunchKernelGGL((k_gemm_b<1, 4, 2>), grid, blk, 0, s, a);
        else if (ng == 2) hipLaunchKernelGGL((k_gemm_b<1, 2, 4>), grid, blk, 0, s, a);
        else hipLaunchKernelGGL((k_gemm_b<1, 1, 8>), grid, blk, 0, s, a);
    }
    hb->launches += 1;
    return p.ks;
}

extern "C" {

mk_status mkb_create(const mk_model_desc* d, int32_t batch, int32_t max_ctx, mkb_handle** out) {
    if (!d || !out || batch < 1 || batch > 64 || max_ctx < 1 || d->n_experts != 0 || !d->layers) return MK_E_INVALID;
    if (d->head_dim != 64 && d->head_dim != 128) return MK_E_INVALID;
    if (d->n_kv_heads < 1 || d->n_q_heads % d->n_kv_heads || d->n_q_heads / d->n_kv_heads > 8) return MK_E_UNSUPPORTED;
    const int h = d->hidden, qd = d->n_q_heads * d->head_dim, kvd = d->n_kv_heads * d->head_dim, f = d->ffn_dim;
    const int R3 = qd + 2 * kvd;
    if (batch == 1) {
        for (int K : {h, qd, f})
            if (K % 512 || K > 8192 || (K & (K - 1))) return MK_E_UNSUPPORTED;
    } else {
        // K a multiple of 256 (whole chunks of the operand stream), every stacked
        // matrix a whole number of row groups (of 64 rows where the stack has 8192 or more)
        for (int K : {h, qd, f})
            if (K % 256) return MK_E_UNSUPPORTED;
        for (int R : {h, qd, kvd, f, d->vocab})
            if (R % 16) return MK_E_UNSUPPORTED;
        for (int R : {R3, h, 2 * f, d->vocab})
            if (R >= 8192 && R % 64) return MK_E_UNSUPPORTED;
        if (R3 >= 8192 && (qd % 64 || kvd % 64)) return MK_E_UNSUPPORTED;
        if (2 * f >= 8192 && f % 64) return MK_E_UNSUPPORTED;
    }
    mkb_handle* hb = new mkb_handle();
    hb->desc = *d;
    hb->layers.assign(d->layers, d->layers + d->n_layers);
    hb->desc.layers = hb->layers.data();
    const int B = batch;
    hb->B = B;
    hb->C = max_ctx;
    // KV chunks per (sequence, group): at most 128 positions each, and at least about
    // 512 workgroups over the step's groups and sequences
    const int by_len = (max_ctx + 127) / 128, by_width = (512 + d->n_kv_heads * B - 1) / (d->n_kv_heads * B);
    hb->S = std::max(1, std::min(64, std::max(by_len, by_width)));
    hb->nb_arg = B == 1 ? 256 : std::max(8, 256 / B);
    size_t gpart = 0;
    if (B > 1) {
        const int Rs[] = {R3, h, 2 * f, h}, Ks[] = {h, qd, h, f};
        for (int i = 0; i < 4; ++i) gpart = std::max(gpart, (size_t)plan_gemm(Rs[i], Ks[i], false).ks * B * Rs[i]);
    }
    const size_t na = (size_t)B * hb->nb_arg;
    const size_t nsplit = B > 1 ? (size_t)B * (h + qd + f) : 0;  // floats holding the bf16 part pairs
    const size_t nf = (size_t)B * ((size_t)h * 4 + R3 + qd * 2 + f + d->vocab) +  // (an upper bound)
                      (size_t)B * d->n_q_heads * hb->S * (d->head_dim + 2) + gpart + nsplit + na * 2 + B + 16 * 20;
    if (hipMalloc(&hb->buf, nf * 4) != hipSuccess) {
        delete hb;
        return MK_E_NOMEM;
    }
    float* p = hb->buf;
    auto take = [&](size_t n) {
        float* r = p;
        p += (n + 15) & ~size_t(15);
        return r;
    };
    // fp32 projection inputs and outputs of the one-sequence path (several sequences
    // use the bf16 part pairs and the K-slice partials instead)
    const size_t one = B == 1 ? 1 : 0;
    hb->x = take((size_t)B * h);
    hb->xn = take(one * h);
    hb->xb = take((size_t)B * h);
    hb->hidden = take((size_t)B * h);
    hb->qkv = take(one * R3);
    hb->q = take((size_t)B * qd);
    hb->a = take(one * qd);
    hb->m = take(one * f);
    hb->lg = take((size_t)B * d->vocab);
    hb->part = take((size_t)B * d->n_q_heads * hb->S * (d->head_dim + 2));
    hb->gpart = take(gpart);
    hb->xs = (uint16_t*)take(B > 1 ? (size_t)B * h : 0);
    hb->as = (uint16_t*)take(B > 1 ? (size_t)B * qd : 0);
    hb->ms = (uint16_t*)take(B > 1 ? (size_t)B * f : 0);
    hb->bv = take(na);
    hb->bi = (int*)take(na);
    hb->next = (int*)take(B);
    const int half = d->head_dim / 2;
    std::vector<float2> tab((size_t)max_ctx * half);
    for (int pos = 0; pos < max_ctx; ++pos)
        for (int j = 0; j < half; ++j) {
            const double ang = (double)pos * std::pow((double)d->rope_theta, -2.0 * j / (double)d->head_dim);
            tab[(size_t)pos * half + j] = make_float2((float)std::cos(ang), (float)std::sin(ang));
        }
    if (hipMalloc(&hb->rope, tab.size() * sizeof(float2)) != hipSuccess ||
        hipMemcpy(hb->rope, tab.data(), tab.size() * sizeof(float2), hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(hb->buf);
        delete hb;
        return MK_E_HIP;
    }
    *out = hb;
    return MK_OK;
}

// One decode step as a sequence of per-op kernels on `stream`.  Same arguments
// as mk_decode_step; when advance != 0 the last kernel also writes the next tokens
// into tokens[] and increments positions[], so a captured graph of this call can
// be replayed step after step.
mk_status mkb_decode_step(mkb_handle* hb, int32_t* tokens, int32_t* positions, void* kv_cache, float* logits,
                          void* stream, int32_t advance) {
    if (!hb || !tokens || !positions || !kv_cache) return MK_E_INVALID;
    const mk_model_desc& d = hb->desc;
    hipStream_t s = (hipStream_t)stream;
    const int B = hb->B, h = d.hidden, D = d.head_dim, nq = d.n_q_heads, nkv = d.n_kv_heads, C = hb->C,
              L = d.n_layers, f = d.ffn_dim, qd = nq * D, kvd = nkv * D;
    const size_t cache_layer = (size_t)B * nkv * C * D;
    uint16_t* kc = (uint16_t*)kv_cache;
    uint16_t* vc = kc + (size_t)L * cache_layer;
    float* lg = logits ? logits : hb->lg;
    const bool one = B == 1;
    hb->launches = 0;
    auto launch = [&](auto kernel, dim3 g, dim3 b, auto... args) {
        hipLaunchKernelGGL(kernel, g, b, 0, s, args...);
        hb->launches += 1;
    };
    launch(k_embed, dim3((h + 255) / 256, B), dim3(256), (const uint16_t*)d.tok_embed, (const int32_t*)tokens, hb->x, h);
    // several sequences: the down-projection slices of the previous layer, added to xb
    // by the next RMSNorm (none before layer 0)
    int ks_down = 0;
    const int rh[1] = {h};
    for (int l = 0; l < L; ++l) {
        const mk_layer_weights& w = d.layers[l];
        // x = xb + down slices; attention RMSNorm
        launch(k_rmsnorm, dim3(B), dim3(1024), (const float*)(ks_down ? hb->xb : hb->x), (const float*)hb->gpart, ks_down,
               hb->x, (const uint16_t*)w.attn_norm, d.rms_eps, one ? hb->xn : (float*)nullptr,
               one ? (uint16_t*)nullptr : hb->xs, h);
        int ks_qkv = 1;
        if (one) {
            gemv_k<EPI_STORE>(h, (const uint16_t*)w.wq, hb->xn, hb->qkv, qd, nullptr, nullptr, s);
            gemv_k<EPI_STORE>(h, (const uint16_t*)w.wk, hb->xn, hb->qkv + qd, kvd, nullptr, nullptr, s);
            gemv_k<EPI_STORE>(h, (const uint16_t*)w.wv, hb->xn, hb->qkv + qd + kvd, kvd, nullptr, nullptr, s);
            hb->launches += 3;
        } else {
            const uint16_t* Wqkv[3] = {(const uint16_t*)w.wq, (const uint16_t*)w.wk, (const uint16_t*)w.wv};
            const int rq[3] = {qd, kvd, kvd};
            ks_qkv = project_b(hb, Wqkv, rq, 3, h, hb->xs, hb->gpart, false, s);
        }
        launch(k_rope_append, dim3(16, B), dim3(256), (const float*)(one ? hb->qkv : hb->gpart), ks_qkv, hb->q,
               (const float2*)hb->rope, (const int32_t*)positions, nq, nkv, D, kc + l * cache_layer,
               vc + l * cache_layer, C);
        const dim3 ag(nkv, hb->S, B), ab(64 * (nq / nkv));
        if (D == 64)
            launch(k_attn_part<64>, ag, ab, (const float*)hb->q, (const uint16_t*)(kc + l * cache_layer),
                   (const uint16_t*)(vc + l * cache_layer), (const int32_t*)positions, nq, nkv, C, hb->S, hb->part);
        else
            launch(k_attn_part<128>, ag, ab, (const float*)hb->q, (const uint16_t*)(kc + l * cache_layer),
                   (const uint16_t*)(vc + l * cache_layer), (const int32_t*)positions, nq, nkv, C, hb->S, hb->part);
        launch(k_attn_merge, dim3(nq, B), dim3(64), (const float*)hb->part, nq, hb->S, D, one ? hb->a : (float*)nullptr,
               one ? (uint16_t*)nullptr : hb->as);
        if (one) {
            // xb = x + Wo a; FFN RMSNorm of xb
            gemv_k<EPI_RESID>(qd, (const uint16_t*)w.wo, hb->a, hb->xb, h, hb->x, nullptr, s);
            hb->launches += 1;
            launch(k_rmsnorm, dim3(1), dim3(1024), (const float*)hb->xb, (const float*)nullptr, 0, hb->xb,
                   (const uint16_t*)w.ffn_norm, d.rms_eps, hb->xn, (uint16_t*)nullptr, h);
            gemv_k<EPI_SILU_MUL>(h, (const uint16_t*)w.w_gate, hb->xn, hb->m, f, nullptr, (const uint16_t*)w.w_up, s);
            gemv_k<EPI_RESID>(f, (const uint16_t*)w.w_down, hb->m, hb->x, h, hb->xb, nullptr, s);
            hb->launches += 2;
        } else {
            const uint16_t* Wo[1] = {(const uint16_t*)w.wo};
            const int ks_o = project_b(hb, Wo, rh, 1, qd, hb->as, hb->gpart, false, s);
            // xb = x + O slices; FFN RMSNorm
            launch(k_rmsnorm, dim3(B), dim3(1024), (const float*)hb->x, (const float*)hb->gpart, ks_o, hb->xb,
                   (const uint16_t*)w.ffn_norm, d.rms_eps, (float*)nullptr, hb->xs, h);
            const uint16_t* Wgu[2] = {(const uint16_t*)w.w_gate, (const uint16_t*)w.w_up};
            const int rgu[2] = {f, f};
            const int ks_gu = project_b(hb, Wgu, rgu, 2, h, hb->xs, hb->gpart, false, s);
            const int n = B * f;
            launch(k_silu_mul, dim3(std::min((n + 255) / 256, 2048)), dim3(256), (const float*)hb->gpart, ks_gu, B, f,
                   hb->ms);
            const uint16_t* Wd[1] = {(const uint16_t*)w.w_down};
            ks_down = project_b(hb, Wd, rh, 1, f, hb->ms, hb->gpart, false, s);
        }
    }
    // x = xb + the last down slices; final RMSNorm
    launch(k_rmsnorm, dim3(B), dim3(1024), (const float*)(ks_down ? hb->xb : hb->x), (const float*)hb->gpart, ks_down,
           hb->x, (const uint16_t*)d.final_norm, d.rms_eps, one ? hb->xn : (float*)nullptr,
           one ? (uint16_t*)nullptr : hb->xs, h);
    const uint16_t* lm = (const uint16_t*)(d.tied_lm_head ? d.tok_embed : d.lm_head);
    if (one) {
        gemv_k<EPI_STORE>(h, lm, hb->xn, lg, d.vocab, nullptr, nullptr, s);
        hb->launches += 1;
    } else {
        const uint16_t* Wl[1] = {lm};
        const int rl[1] = {d.vocab};
        project_b(hb, Wl, rl, 1, h, hb->xs, lg, true, s);
    }
    launch(k_argmax1, dim3(hb->nb_arg, B), dim3(256), (const float*)lg, d.vocab, hb->bv, hb->bi);
    launch(k_argmax2, dim3(B), dim3(256), (const float*)hb->bv, (const int*)hb->bi, hb->nb_arg, hb->next,
           (const float*)hb->x, hb->hidden, h, advance ? tokens : (int32_t*)nullptr,
           advance ? positions : (int32_t*)nullptr);
    return hipGetLastError() == hipSuccess ? MK_OK : MK_E_HIP;
}

const int32_t* mkb_next_tokens(const mkb_handle* hb) { return hb ? hb->next : nullptr; }
const float* mkb_hidden_out(const mkb_handle* hb) { return hb ? hb->hidden : nullptr; }
int32_t mkb_launches_per_step(const mkb_handle* hb) { return hb ? hb->launches : 0; }

void mkb_destroy(mkb_handle* hb) {
    if (!hb) return;
    (void)hipDeviceSynchronize();
    (void)hipFree(hb->buf);
    (void)hipFree(hb->rope);
    delete hb;
}

}  // extern "C"
