// One-kernel-per-op HIP baseline of the same decode step, for comparison with
// the megakernel: every operator is its own launch and every launch boundary is
// a device-wide barrier, the execution model the pages contrast the megakernel
// with (Hazy Research megakernel news page, section 3, "problems of existing
// methods": hundreds of short kernels, launch cost, idle SMs in the tail of
// each kernel, waiting for weights after each launch; cloud.baidu.com
// explainer, section 3: per-operator kernels write their intermediates to
// memory).  Same arithmetic as the megakernel (bf16 weights, fp32 activations
// and accumulation), independent code.
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

// x = embedding row of the token
__global__ void k_embed(const uint16_t* E, const int32_t* tok, float* x, int h) {
    const uint16_t* row = E + (size_t)tok[0] * h;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < h; i += gridDim.x * blockDim.x) x[i] = bf(row[i]);
}

// xn = x * g / sqrt(mean(x^2) + eps); one workgroup of 256 threads
__global__ void __launch_bounds__(256) k_rmsnorm(const float* x, const uint16_t* g, float eps, float* xn, int h) {
    __shared__ float part[4];
    float ss = 0.f;
    for (int i = threadIdx.x; i < h; i += 256) ss += x[i] * x[i];
    ss = warp_sum(ss);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float r = 1.0f / sqrtf((part[0] + part[1] + part[2] + part[3]) / (float)h + eps);
    for (int i = threadIdx.x; i < h; i += 256) xn[i] = x[i] * r * bf(g[i]);
}

// y[r] = W[r,:] . x (+ epilogue): each wave computes R consecutive rows, each lane
// 8 columns per 512-column stride; K is a multiple of 512.
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

// RoPE on q and k (pairs j, j + d/2 of each head) and K/V append (bf16) at slot pos
__global__ void k_rope_append(float* q, float* k, const float* v, const float2* rope, const int32_t* pos, int nq,
                              int nkv, int d, uint16_t* kc, uint16_t* vc, int C) {
    const int half = d / 2;
    const int P = pos[0];
    const int n = (nq + nkv) * half;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n + nkv * d; i += gridDim.x * blockDim.x) {
        if (i < n) {
            const int hd = i / half, j = i % half;
            float* u = hd < nq ? q + (size_t)hd * d : k + (size_t)(hd - nq) * d;
            const float2 cs = rope[(size_t)P * half + j];
            const float lo = u[j], hi = u[j + half];
            const float a = lo * cs.x - hi * cs.y, b = lo * cs.y + hi * cs.x;
            u[j] = a;
            u[j + half] = b;
            if (hd >= nq) {
                const int g = hd - nq;
                kc[((size_t)g * C + P) * d + j] = to_bf16(a);
                kc[((size_t)g * C + P) * d + j + half] = to_bf16(b);
            }
        } else {
            const int t = i - n, g = t / d, e = t % d;
            vc[((size_t)g * C + P) * d + e] = to_bf16(v[t]);
        }
    }
}

// Attention partial over chunk blockIdx.y of the context, one wave per query head.
// Writes (m, l, o[d]) to part[head][chunk].
template <int D>
__global__ void __launch_bounds__(64) k_attn_part(const float* q, const uint16_t* kc, const uint16_t* vc,
                                                  const int32_t* pos, int grp, int C, int splits, float* part) {
    const int hq = blockIdx.x, c = blockIdx.y, lane = threadIdx.x;
    const int g = hq / grp;
    const int n = pos[0] + 1;
    const int lc = (n + splits - 1) / splits;
    const int p0 = min(n, c * lc), p1 = min(n, p0 + lc);
    const uint16_t* K = kc + (size_t)g * C * D;
    const uint16_t* V = vc + (size_t)g * C * D;
    __shared__ float qs[D];
    __shared__ float ws[64];
    for (int t = lane; t < D; t += 64) qs[t] = q[(size_t)hq * D + t];
    __syncthreads();
    const float scale = 1.0f / sqrtf((float)D);
    float M = -INFINITY, L = 0.f, o[D / 64];
    for (int e = 0; e < D / 64; ++e) o[e] = 0.f;
    for (int b0 = p0; b0 < p1; b0 += 64) {
        const int p = b0 + lane;
        float s = -INFINITY;
        if (p < p1) {
            const uint4* kr = (const uint4*)(K + (size_t)p * D);
            float a = 0.f;
            for (int cc = 0; cc < D / 8; ++cc) {
                const uint4 w = kr[cc];
                const float* qq = qs + cc * 8;
                a += bflo(w.x) * qq[0] + bfhi(w.x) * qq[1] + bflo(w.y) * qq[2] + bfhi(w.y) * qq[3] +
                     bflo(w.z) * qq[4] + bfhi(w.z) * qq[5] + bflo(w.w) * qq[6] + bfhi(w.w) * qq[7];
            }
            s = a * scale;
        }
        const float mn = fmaxf(M, warp_max(s));
        const float corr = __expf(M - mn);
        const float e = p < p1 ? __expf(s - mn) : 0.f;
        L = L * corr + warp_sum(e);
        M = mn;
        ws[lane] = e;
        __syncthreads();
        for (int ee = 0; ee < D / 64; ++ee) o[ee] *= corr;
        const int nb = min(64, p1 - b0);
        for (int r = 0; r < nb; ++r) {
            const float wgt = ws[r];
            for (int ee = 0; ee < D / 64; ++ee) o[ee] = fmaf(wgt, bf(V[(size_t)(b0 + r) * D + lane + 64 * ee]), o[ee]);
        }
        __syncthreads();
    }
    float* dst = part + ((size_t)hq * splits + c) * (D + 2);
    if (lane == 0) {
        dst[0] = M;
        dst[1] = L;
    }
    for (int ee = 0; ee < D / 64; ++ee) dst[2 + lane + 64 * ee] = o[ee];
}

// Merge of the chunk partials of each query head: a[head][t]
__global__ void k_attn_merge(const float* part, int splits, int D, float* a) {
    const int hq = blockIdx.x;
    const float* src = part + (size_t)hq * splits * (D + 2);
    float Mx = -INFINITY;
    for (int c = 0; c < splits; ++c) Mx = fmaxf(Mx, src[c * (D + 2)]);
    for (int t = threadIdx.x; t < D; t += blockDim.x) {
        float den = 0.f, num = 0.f;
        for (int c = 0; c < splits; ++c) {
            const float m = src[c * (D + 2)];
            const float sc = m == -INFINITY ? 0.f : __expf(m - Mx);
            den += sc * src[c * (D + 2) + 1];
            num += sc * src[c * (D + 2) + 2 + t];
        }
        a[(size_t)hq * D + t] = num / den;
    }
}

// argmax over logits: stage 1 per block (value, lowest index), stage 2 over the blocks
__global__ void __launch_bounds__(256) k_argmax1(const float* v, int n, float* bv, int* bi) {
    __shared__ float sv[256];
    __shared__ int si[256];
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
        if (threadIdx.x < s) {
            const float ov = sv[threadIdx.x + s];
            const int oi = si[threadIdx.x + s];
            if (ov > sv[threadIdx.x] || (ov == sv[threadIdx.x] && oi < si[threadIdx.x])) {
                sv[threadIdx.x] = ov;
                si[threadIdx.x] = oi;
            }
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        bv[blockIdx.x] = sv[0];
        bi[blockIdx.x] = si[0];
    }
}
__global__ void k_argmax2(const float* bv, const int* bi, int nb, int* next, const float* x, float* hidden, int h,
                          int32_t* tok_out, int32_t* pos_inout) {
    if (threadIdx.x == 0) {
        float best = -INFINITY;
        int idx = 0x7fffffff;
        for (int b = 0; b < nb; ++b)
            if (bv[b] > best || (bv[b] == best && bi[b] < idx)) {
                best = bv[b];
                idx = bi[b];
            }
        next[0] = idx;
        if (tok_out) tok_out[0] = idx;
        if (pos_inout) pos_inout[0] += 1;
    }
    for (int i = threadIdx.x; i < h; i += blockDim.x) hidden[i] = x[i];
}

}  // namespace mkb

using namespace mkb;

struct mkb_handle {
    mk_model_desc desc;
    std::vector<mk_layer_weights> layers;
    int C = 0, S = 8;
    float* buf = nullptr;  // x, xn, q, k, v, a, h1, m, logits scratch, part, argmax
    float *x, *xn, *q, *k, *v, *a, *xb, *m, *lg, *part, *bv, *hidden;
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
bool gemv_k(int K, const uint16_t* W, const float* x, float* y, int rows, const float* aux, const uint16_t* W2,
            hipStream_t s) {
    switch (K) {
        case 512: gemv<512, EPI>(W, x, y, rows, aux, W2, s); return true;
        case 1024: gemv<1024, EPI>(W, x, y, rows, aux, W2, s); return true;
        case 2048: gemv<2048, EPI>(W, x, y, rows, aux, W2, s); return true;
        case 4096: gemv<4096, EPI>(W, x, y, rows, aux, W2, s); return true;
        case 8192: gemv<8192, EPI>(W, x, y, rows, aux, W2, s); return true;
        default: return false;
    }
}

}  // namespace

extern "C" {

mk_status mkb_create(const mk_model_desc* d, int32_t batch, int32_t max_ctx, mkb_handle** out) {
    if (!d || !out || batch != 1 || max_ctx < 1 || d->n_experts != 0) return MK_E_INVALID;
    if (d->head_dim != 64 && d->head_dim != 128) return MK_E_INVALID;
    const int h = d->hidden, qd = d->n_q_heads * d->head_dim, kvd = d->n_kv_heads * d->head_dim;
    for (int K : {h, qd, d->ffn_dim})
        if (K % 512 || K > 8192 || (K & (K - 1))) return MK_E_UNSUPPORTED;
    mkb_handle* hb = new mkb_handle();
    hb->desc = *d;
    hb->layers.assign(d->layers, d->layers + d->n_layers);
    hb->desc.layers = hb->layers.data();
    hb->C = max_ctx;
    hb->S = std::max(1, std::min(16, (max_ctx + 255) / 256));
    const size_t nb = 256;
    const size_t nf = (size_t)h * 3 + qd * 2 + kvd * 2 + d->ffn_dim + d->vocab +
                      (size_t)d->n_q_heads * hb->S * (d->head_dim + 2) + nb + h + 64;
    if (hipMalloc(&hb->buf, nf * 4 + nb * 4 + 64) != hipSuccess) {
        delete hb;
        return MK_E_NOMEM;
    }
    float* p = hb->buf;
    auto take = [&](size_t n) {
        float* r = p;
        p += (n + 15) & ~size_t(15);
        return r;
    };
    hb->x = take(h);
    hb->xn = take(h);
    hb->xb = take(h);
    hb->q = take(qd);
    hb->a = take(qd);
    hb->k = take(kvd);
    hb->v = take(kvd);
    hb->m = take(d->ffn_dim);
    hb->lg = take(d->vocab);
    hb->part = take((size_t)d->n_q_heads * hb->S * (d->head_dim + 2));
    hb->bv = take(nb);
    hb->hidden = take(h);
    hb->bi = (int*)take(nb);
    hb->next = (int*)take(16);
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
// as mk_decode_step; when advance != 0 the last kernel also writes the next token
// into tokens[0] and increments positions[0], so a captured graph of this call
// can be replayed step after step.
mk_status mkb_decode_step(mkb_handle* hb, int32_t* tokens, int32_t* positions, void* kv_cache, float* logits,
                          void* stream, int32_t advance) {
    if (!hb || !tokens || !positions || !kv_cache) return MK_E_INVALID;
    const mk_model_desc& d = hb->desc;
    hipStream_t s = (hipStream_t)stream;
    const int h = d.hidden, D = d.head_dim, nq = d.n_q_heads, nkv = d.n_kv_heads, C = hb->C, L = d.n_layers;
    const size_t cache_layer = (size_t)nkv * C * D;
    uint16_t* kc = (uint16_t*)kv_cache;
    uint16_t* vc = kc + (size_t)L * cache_layer;
    float* lg = logits ? logits : hb->lg;
    hipLaunchKernelGGL(k_embed, dim3((h + 255) / 256), dim3(256), 0, s, (const uint16_t*)d.tok_embed, tokens, hb->x, h);
    for (int l = 0; l < L; ++l) {
        const mk_layer_weights& w = d.layers[l];
        hipLaunchKernelGGL(k_rmsnorm, dim3(1), dim3(256), 0, s, hb->x, (const uint16_t*)w.attn_norm, d.rms_eps, hb->xn, h);
        gemv_k<EPI_STORE>(h, (const uint16_t*)w.wq, hb->xn, hb->q, nq * D, nullptr, nullptr, s);
        gemv_k<EPI_STORE>(h, (const uint16_t*)w.wk, hb->xn, hb->k, nkv * D, nullptr, nullptr, s);
        gemv_k<EPI_STORE>(h, (const uint16_t*)w.wv, hb->xn, hb->v, nkv * D, nullptr, nullptr, s);
        hipLaunchKernelGGL(k_rope_append, dim3(8), dim3(256), 0, s, hb->q, hb->k, hb->v, hb->rope, positions, nq, nkv, D,
                           kc + l * cache_layer, vc + l * cache_layer, C);
        if (D == 64)
            hipLaunchKernelGGL(k_attn_part<64>, dim3(nq, hb->S), dim3(64), 0, s, hb->q, kc + l * cache_layer,
                               vc + l * cache_layer, positions, nq / nkv, C, hb->S, hb->part);
        else
            hipLaunchKernelGGL(k_attn_part<128>, dim3(nq, hb->S), dim3(64), 0, s, hb->q, kc + l * cache_layer,
                               vc + l * cache_layer, positions, nq / nkv, C, hb->S, hb->part);
        hipLaunchKernelGGL(k_attn_merge, dim3(nq), dim3(64), 0, s, hb->part, hb->S, D, hb->a);
        gemv_k<EPI_RESID>(nq * D, (const uint16_t*)w.wo, hb->a, hb->xb, h, hb->x, nullptr, s);
        hipLaunchKernelGGL(k_rmsnorm, dim3(1), dim3(256), 0, s, hb->xb, (const uint16_t*)w.ffn_norm, d.rms_eps, hb->xn, h);
        gemv_k<EPI_SILU_MUL>(h, (const uint16_t*)w.w_gate, hb->xn, hb->m, d.ffn_dim, nullptr, (const uint16_t*)w.w_up, s);
        gemv_k<EPI_RESID>(d.ffn_dim, (const uint16_t*)w.w_down, hb->m, hb->x, h, hb->xb, nullptr, s);
    }
    hipLaunchKernelGGL(k_rmsnorm, dim3(1), dim3(256), 0, s, hb->x, (const uint16_t*)d.final_norm, d.rms_eps, hb->xn, h);
    const uint16_t* lm = (const uint16_t*)(d.tied_lm_head ? d.tok_embed : d.lm_head);
    gemv_k<EPI_STORE>(h, lm, hb->xn, lg, d.vocab, nullptr, nullptr, s);
    hipLaunchKernelGGL(k_argmax1, dim3(256), dim3(256), 0, s, lg, d.vocab, hb->bv, hb->bi);
    hipLaunchKernelGGL(k_argmax2, dim3(1), dim3(256), 0, s, hb->bv, hb->bi, 256, hb->next, hb->x, hb->hidden, h,
                       advance ? tokens : nullptr, advance ? positions : nullptr);
    return hipGetLastError() == hipSuccess ? MK_OK : MK_E_HIP;
}

const int32_t* mkb_next_tokens(const mkb_handle* hb) { return hb ? hb->next : nullptr; }
const float* mkb_hidden_out(const mkb_handle* hb) { return hb ? hb->hidden : nullptr; }

void mkb_destroy(mkb_handle* hb) {
    if (!hb) return;
    (void)hipDeviceSynchronize();
    (void)hipFree(hb->buf);
    (void)hipFree(hb->rope);
    delete hb;
}

}  // extern "C"
