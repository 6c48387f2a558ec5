// The prompt (prefill) megakernel's operations, included by megakernel.hip after the
// decode operations whose helpers they share (LDS ring, barriers, event waits, the
// several-sequence GEMV for the LM head).
//
// One launch runs the T tokens of one sequence's prompt through the decoder (the
// prefill pass that the knowledge-base digest "megakernel boundary selection" defines
// in its list of first-used concepts, and to which its planner gives Llama-1B a
// megakernel of its own, Figure 4).  With T tokens every projection is a GEMM, so its
// tasks are GEMM tiles on the matrix cores: a task holds `rows` output rows x a block
// of 64 or 128 tokens, streams its weight tile through the LDS pages once, and reads the
// token operands (two bf16 parts per fp32 input, as the several-sequence decode path)
// from L2.  Buffers of a prompt handle:
//   p.acc  residual rows, fp32 [Tp][h] each (Tp = T rounded up to 16): R_b the input of a layer
//          (after the last layer: the hidden output), R_a after its attention; then the K-slice
//          partial outputs of the O-projection [S_o][Tp][h] and of the down projection [S_d][Tp][h],
//          which the next RMSNorm tasks add to the residual (no atomics)
//   p.xop  matrix-core B operands in units of (token group of 16, 32-column block):
//          [part][64 lanes][8 bf16] = 2 KiB, lane = token % 16 + 16 ((column % 32) / 8);
//          X [ntg][h/32] normalised input of QKV or gate/up, O [ntg][nq d/32] attention
//          output, M [ntg][f/32] SiLU(gate) * up, LM [h/32] the final normalised last
//          token (column 0; the other columns stay zero)
//   p.q    query operands [ntg][nq][d/32][part][64][8]
// Every cross-workgroup datum is written and read with device-scope (sc1) accesses,
// and a producer's stores are acknowledged before it signals (as in the decode path).

__device__ __forceinline__ int pf_ntg(CParams& p) { return (p.T.pf_T + 15) / 16; }
__device__ __forceinline__ uint16_t* pf_x(CParams& p) { return p.xop; }
__device__ __forceinline__ uint16_t* pf_o(CParams& p) { return p.xop + (size_t)pf_ntg(p) * (p.T.h / 32) * 1024; }
__device__ __forceinline__ uint16_t* pf_m(CParams& p) {
    return pf_o(p) + (size_t)pf_ntg(p) * (p.T.nq * p.T.d / 32) * 1024;
}
__device__ __forceinline__ uint16_t* pf_lm(CParams& p) { return pf_m(p) + (size_t)pf_ntg(p) * (p.T.f / 32) * 1024; }
__device__ __forceinline__ size_t pf_rows(CParams& p) { return (size_t)pf_ntg(p) * 16 * p.T.h; }  // floats per [Tp][h]
__device__ __forceinline__ float* pf_ra(CParams& p) { return p.acc; }
__device__ __forceinline__ float* pf_rb(CParams& p) { return p.acc + pf_rows(p); }
// K-slice partial outputs of the O-projection (slice s) and of the down projection
__device__ __forceinline__ float* pf_po(CParams& p, int s) { return p.acc + (2 + (size_t)s) * pf_rows(p); }
__device__ __forceinline__ float* pf_pd(CParams& p, int s) {
    return p.acc + (2 + (size_t)p.T.pf_slices[1] + (size_t)s) * pf_rows(p);
}

// byte offset of (token group tg, column block kb, part pt, lane) in a region of nkb column blocks
__device__ __forceinline__ uint32_t pf_unit(uint32_t tg, uint32_t nkb, uint32_t kb, uint32_t pt, uint32_t lane) {
    return (((tg * nkb + kb) * 2u + pt) * 64u + lane) * 16u;
}
// the two parts of 4 consecutive values (one lane's 4 rows of a result block) as 8-byte words
__device__ __forceinline__ void split4(const float* v, u32x2v& hi, u32x2v& lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split2(v[i], h[i], l[i]);
    hi = u32x2v{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
    lo = u32x2v{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
}
__device__ __forceinline__ void st8_dev(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2v v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 16);
}

// RMSNorm task of one token (short prompts: one task per token spreads the phase over as many
// workgroups as there are tokens): compute wave w takes columns w h/4 .. (w + 1) h/4 - 1, eight
// per lane; the four waves' sums of squares meet in LDS.  Same arithmetic and summation order as
// the four-token task.
__device__ __forceinline__ bool pnorm_token(const Params* pp, const Task& k, Ctx& c, const uint16_t* gp) {
    CParams& p = P(pp);
    const int lane = c.lane, wave = c.wave;
    const int h = p.T.h, Tn = p.T.pf_T, l = k.layer, kind = k.part, nkb = h / 32;
    const int tok = (int)k.seq, cw = h / NCW, c0 = wave * cw + lane * 8;
    const bool act = lane * 8 < cw && tok < Tn;
    const uint4 gw = act ? gld_u4(gp + c0) : make_uint4(0, 0, 0, 0);
    if (!await_inputs(pp, k, c)) return false;
    tmark(c, 0);
    const uint32_t rbytes = (uint32_t)(pf_rows(p) * 4);
    const float* base = kind == 1 ? pf_rb(p) : pf_ra(p);
    const int nsl = kind == 1 ? p.T.pf_slices[1] : p.T.pf_slices[3];
    const float* part0 = kind == 1 ? pf_po(p, 0) : pf_pd(p, 0);
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = 0.f;
    if (act) {
        if (kind == 0 && l == 0) {
            const int id = gld(S.args.tokens + tok);
            const uint4 v = gld_u4((const uint16_t*)(p.w + p.lay.embed) + (size_t)id * h + c0);
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[2 * e] = bf16lo(w4[e]);
                x[2 * e + 1] = bf16hi(w4[e]);
            }
        } else {
            // the residual and the partials, all loads in flight at once, added in slice order
            u32x4 a[PF_MAX_SLICES + 1], b[PF_MAX_SLICES + 1];
            const uint32_t off = (uint32_t)(tok * h + c0) * 4u;
#pragma unroll
            for (int q = 0; q <= PF_MAX_SLICES; ++q) {
                if (q > nsl) break;
                const __amdgpu_buffer_rsrc_t r = dev_rsrc(q == 0 ? base : part0 + (size_t)(q - 1) * pf_rows(p), rbytes);
                a[q] = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16);
                b[q] = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 16);
            }
#pragma unroll
            for (int q = 0; q <= PF_MAX_SLICES; ++q) {
                if (q > nsl) break;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[e] += __uint_as_float(a[q][e]);
                    x[4 + e] += __uint_as_float(b[q][e]);
                }
            }
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
    ss = wave_sum(ss);
    // the four waves' sums (a slot per task parity: a wave a task ahead cannot overwrite them)
    if (lane == 0) S.ssqb[wave][c.t & 1u] = ss;
    if (!cbarrier(pp, c, k.id)) return false;
    ss = (S.ssqb[0][c.t & 1u] + S.ssqb[1][c.t & 1u]) + (S.ssqb[2][c.t & 1u] + S.ssqb[3][c.t & 1u]);
    tmark(c, 1);
    if (!act) return true;
    const float rs = 1.0f / sqrtf(ss / (float)h + p.eps);
    const __amdgpu_buffer_rsrc_t dst = dev_rsrc(kind == 1 ? pf_ra(p) : pf_rb(p), rbytes);
    const uint32_t off = (uint32_t)(tok * h + c0) * 4u;
    __builtin_amdgcn_raw_buffer_store_b128(
        u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])}, dst, off, 0,
        16);
    __builtin_amdgcn_raw_buffer_store_b128(
        u32x4{__float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]), __float_as_uint(x[7])}, dst,
        off + 16, 0, 16);
    if (kind == 2 && tok != Tn - 1) return true;
    const int tg = kind == 2 ? 0 : tok / 16, n = kind == 2 ? 0 : tok % 16;
    const __amdgpu_buffer_rsrc_t reg =
        dev_rsrc(kind == 2 ? pf_lm(p) : pf_x(p), (uint32_t)(kind == 2 ? 1 : pf_ntg(p)) * nkb * 2048u);
    const uint32_t g4[4] = {gw.x, gw.y, gw.z, gw.w};
    float y[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        y[2 * e] = x[2 * e] * rs * bf16lo(g4[e]);
        y[2 * e + 1] = x[2 * e + 1] * rs * bf16hi(g4[e]);
    }
    u32x4v hi, lo;
    split8(y, hi, lo);
    const uint32_t ln = (uint32_t)(n + 16 * ((c0 % 32) / 8));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, hi), reg,
                                           pf_unit((uint32_t)tg, (uint32_t)nkb, (uint32_t)(c0 / 32), 0, ln), 0, 16);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, lo), reg,
                                           pf_unit((uint32_t)tg, (uint32_t)nkb, (uint32_t)(c0 / 32), 1, ln), 0, 16);
    return true;
}

// RMSNorm tasks of 4 tokens (compute wave w: token 4 q + w; a lane holds columns 512 j + 8 lane
// .. + 7), or of one (nrows = 1: pnorm_token).  Each first completes the residual: kind 0 (the attention input of layer l) x = R_a +
// the previous layer's down partials (layer 0: the embedding row) -> R_b; kind 1 (the FFN input)
// x = R_b + this layer's O-projection partials -> R_a; kind 2 (after the last layer) x = R_a + the
// down partials -> R_b, the hidden output.  Then x is normalised into the X operands (kind 2: of
// the last prompt token only, into the LM operands).  Tokens past the prompt write zero operands.
__device__ __noinline__ bool op_pnorm(const Params* pp, uint32_t slot_, uint32_t page0, uint32_t t_, uint32_t epoch_) {
    const Task k = fifo_task(slot_);
    Ctx c = make_ctx(t_, epoch_);
    CParams& p = P(pp);
    (void)page0;
    const int lane = c.lane, wave = c.wave;
    const int h = p.T.h, L = p.T.L, Tn = p.T.pf_T, l = k.layer, kind = k.part;
    const int nkb = h / 32, NJ = h / 512;
    const uint16_t* gp = gains(p, kind == 0 ? 2 * l : kind == 1 ? 2 * l + 1 : 2 * L);
    if (k.nrows == 1) return pnorm_token(pp, k, c, gp);
    const int tok = (int)k.seq * 4 + wave;
    const bool valid = tok < Tn;
    uint4 gw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (j < NJ) gw[j] = gld_u4(gp + j * 512 + lane * 8);
    if (!await_inputs(pp, k, c)) return false;
    tmark(c, 0);
    const uint32_t rbytes = (uint32_t)(pf_rows(p) * 4);
    // the residual so far and the partials to add (nsl of them, all [Tp][h])
    const float* base = kind == 1 ? pf_rb(p) : pf_ra(p);
    const int nsl = kind == 1 ? p.T.pf_slices[1] : p.T.pf_slices[3];
    const float* part0 = kind == 1 ? pf_po(p, 0) : pf_pd(p, 0);
    const bool from_emb = kind == 0 && l == 0;
    float x[4][8];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[j][e] = 0.f;
    if (valid) {
        if (from_emb) {
            const int id = gld(S.args.tokens + tok);
            const uint16_t* emb = (const uint16_t*)(p.w + p.lay.embed) + (size_t)id * h;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (j >= NJ) break;
                const uint4 v = gld_u4(emb + j * 512 + lane * 8);
                const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[j][2 * e] = bf16lo(w4[e]);
                    x[j][2 * e + 1] = bf16hi(w4[e]);
                }
            }
        } else {
            // the residual and up to PF_MAX_SLICES partials, added in slice order; each half of the
            // row's columns with all of its loads in flight at once
#pragma unroll
            for (int jh = 0; jh < 2; ++jh) {
                if (2 * jh >= NJ) break;
                u32x4 a[PF_MAX_SLICES + 1][2], b[PF_MAX_SLICES + 1][2];
#pragma unroll
                for (int q = 0; q <= PF_MAX_SLICES; ++q) {
                    if (q > nsl) break;
                    const __amdgpu_buffer_rsrc_t r =
                        dev_rsrc(q == 0 ? base : part0 + (size_t)(q - 1) * pf_rows(p), rbytes);
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj) {
                        const int j = 2 * jh + jj;
                        if (j >= NJ) break;
                        const uint32_t off = (uint32_t)(tok * h + j * 512 + lane * 8) * 4u;
                        a[q][jj] = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16);
                        b[q][jj] = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 16);
                    }
                }
#pragma unroll
                for (int q = 0; q <= PF_MAX_SLICES; ++q) {
                    if (q > nsl) break;
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj) {
                        const int j = 2 * jh + jj;
                        if (j >= NJ) break;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            x[j][e] += __uint_as_float(a[q][jj][e]);
                            x[j][4 + e] += __uint_as_float(b[q][jj][e]);
                        }
                    }
                }
            }
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(x[j][e], x[j][e], ss);
    ss = wave_sum(ss);
    tmark(c, 1);
    const float rs = 1.0f / sqrtf(ss / (float)h + p.eps);
    // the completed residual
    const __amdgpu_buffer_rsrc_t dst = dev_rsrc(kind == 1 ? pf_ra(p) : pf_rb(p), rbytes);
    if (valid) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j >= NJ) break;
            const uint32_t off = (uint32_t)(tok * h + j * 512 + lane * 8) * 4u;
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{__float_as_uint(x[j][0]), __float_as_uint(x[j][1]),
                                                         __float_as_uint(x[j][2]), __float_as_uint(x[j][3])},
                                                   dst, off, 0, 16);
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{__float_as_uint(x[j][4]), __float_as_uint(x[j][5]),
                                                         __float_as_uint(x[j][6]), __float_as_uint(x[j][7])},
                                                   dst, off + 16, 0, 16);
        }
    }
    // the normalised row as matrix-core operands
    if (kind == 2 && tok != Tn - 1) return true;
    const int tg = kind == 2 ? 0 : tok / 16, n = kind == 2 ? 0 : tok % 16;
    const __amdgpu_buffer_rsrc_t reg =
        dev_rsrc(kind == 2 ? pf_lm(p) : pf_x(p), (uint32_t)(kind == 2 ? 1 : pf_ntg(p)) * nkb * 2048u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (j >= NJ) break;
        const int c0 = j * 512 + lane * 8;
        const uint32_t g4[4] = {gw[j].x, gw[j].y, gw[j].z, gw[j].w};
        float y[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            y[2 * e] = x[j][2 * e] * rs * bf16lo(g4[e]);
            y[2 * e + 1] = x[j][2 * e + 1] * rs * bf16hi(g4[e]);
        }
        u32x4v hi, lo;
        split8(y, hi, lo);
        const uint32_t ln = (uint32_t)(n + 16 * ((c0 % 32) / 8));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, hi), reg,
                                               pf_unit((uint32_t)tg, (uint32_t)nkb, (uint32_t)(c0 / 32), 0, ln), 0, 16);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, lo), reg,
                                               pf_unit((uint32_t)tg, (uint32_t)nkb, (uint32_t)(c0 / 32), 1, ln), 0, 16);
    }
    return true;
}

// GEMM tile of projection OPK: rows x (64 NGW tokens) over one K slice.  The weight tile
// arrives page by page (RG = rows / 16 row groups x 16 / RG column blocks per page);
// every compute wave reads the whole page and multiplies it with its own token groups
// (tgw, tgw + 4), whose two-part B operands it loads from L2 one page ahead.  Results:
// acc[rg][j] holds rows 16 rg + 4 (lane / 16) + i, token 16 (tgw + 4 j) + lane % 16.
template <int OPK, int RG, int NGW>
__device__ __noinline__ bool op_pgemm(const Params* pp, uint32_t slot_, uint32_t page0, uint32_t t_, uint32_t epoch_) {
    constexpr int KBP = 16 / RG;
    static_assert(RG == 4 || RG == 8, "prompt GEMM tiles have 64 or 128 rows");
    page0 = uni(page0);  // wave-uniform (a call passes it in a vector register): scalar page waits
    const Task k = fifo_task(slot_);
    Ctx c = make_ctx(t_, epoch_);
    CParams& p = P(pp);
    const int lane = c.lane, wave = c.wave, n = lane % 16, kq = lane / 16;
    const int h = p.T.h, Tn = p.T.pf_T, l = k.layer, D = p.T.d, ntg = pf_ntg(p);
    const int nkb = OPK == OP_PQKV || OPK == OP_PGU ? h / 32 : OPK == OP_POPROJ ? p.T.nq * D / 32 : p.T.f / 32;
    const uint16_t* R = OPK == OP_PQKV || OPK == OP_PGU ? pf_x(p) : OPK == OP_POPROJ ? pf_o(p) : pf_m(p);
    const __amdgpu_buffer_rsrc_t br = dev_rsrc(R, (uint32_t)(ntg * nkb) * 2048u);
    const uint32_t npages = k.wbytes / PAGE;
    const uint32_t kb0 = k.part * npages * KBP;  // first column block of this K slice
    const int tgw = (int)k.seq * 4 * NGW + wave;  // this wave's first token group (then + 4)
    if (!await_inputs(pp, k, c)) return false;
    tmark(c, 0);
    const bool trace_pages = wave == 0 && c.tr;
    f32x4v acc[RG][NGW];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int j = 0; j < NGW; ++j) acc[rg][j] = f32x4v{0.f, 0.f, 0.f, 0.f};
    // B operands of page pg (token groups past the prompt's last read zeros: past the region)
    auto load_b = [&](u32x4v (&b)[NGW][KBP][NPART], uint32_t pg) {
#pragma unroll
        for (int j = 0; j < NGW; ++j)
#pragma unroll
            for (int kb = 0; kb < KBP; ++kb)
#pragma unroll
                for (int pt = 0; pt < NPART; ++pt)
                    b[j][kb][pt] = __builtin_bit_cast(
                        u32x4v, __builtin_amdgcn_raw_buffer_load_b128(
                                    br,
                                    pf_unit((uint32_t)(tgw + 4 * j), (uint32_t)nkb, kb0 + pg * KBP + (uint32_t)kb,
                                            (uint32_t)pt, (uint32_t)lane),
                                    0, 16));
    };
    // one page: the B operands of the page after next are issued first (two pages of loads stay in
    // flight during the products); the page's A blocks are read one column block at a time.  The
    // prefetch is unconditional (past the last page it reads other columns of the region, or zeros
    // past its end, never used): a conditional one would make the compiler wait for every load.
    auto page = [&](uint32_t s, const u32x4v (&bc)[NGW][KBP][NPART], u32x4v (&bn)[NGW][KBP][NPART]) -> bool {
        load_b(bn, s + 2);
        if (!page_acquire_tr(pp, page0 + s, k.id, trace_pages, lane)) return false;
        if (trace_pages && lane == 0) lds_st(S.tm[2], (uint32_t)rtc());
        const uint32_t slot = (page0 + s) % NPAGES;
#pragma unroll
        for (int kb = 0; kb < KBP; ++kb) {
            u32x4v a[RG];
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) a[rg] = *(const u32x4v*)&ring[slot][(kb * RG + rg) * 1024 + lane * 16];
            // parts outermost: an accumulator's consecutive products are RG * NGW issues apart
#pragma unroll
            for (int pt = 0; pt < NPART; ++pt)
#pragma unroll
                for (int rg = 0; rg < RG; ++rg)
#pragma unroll
                    for (int j = 0; j < NGW; ++j)
                        acc[rg][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8v, a[rg]), __builtin_bit_cast(bf16x8v, bc[j][kb][pt]),
                            acc[rg][j], 0, 0, 0);
        }
        page_release(page0 + s, lane);
        return true;
    };
    u32x4v b0[NGW][KBP][NPART], b1[NGW][KBP][NPART], b2[NGW][KBP][NPART];
    load_b(b0, 0);
    load_b(b1, 1);
    for (uint32_t s = 0; s < npages; s += 3) {
        if (!page(s, b0, b2)) return false;
        if (s + 1 < npages && !page(s + 1, b1, b0)) return false;
        if (s + 2 < npages && !page(s + 2, b2, b1)) return false;
    }
    tmark(c, 1);
    const int32_t pos0 = (int32_t)uni((uint32_t)S.args.pos0);
#pragma unroll
    for (int j = 0; j < NGW; ++j) {
        const int tg = tgw + 4 * j, tok = tg * 16 + n;
        if (tg >= ntg) break;
        if constexpr (OPK == OP_PQKV) {
            if (tok >= Tn) continue;
            const int nq = p.T.nq, nkv = p.T.nkv, pos = pos0 + tok;
#pragma unroll
            for (int hb = 0; hb < RG / 4; ++hb) {
                const int head = ((int)k.row0 + 64 * hb) / 64;  // head slot: q heads, then k, then v
                const bool is_q = head < nq, is_k = !is_q && head < nq + nkv;
#pragma unroll
                for (int rl = 0; rl < 2; ++rl) {
                    // pairs (jd, jd + 32), jd = 16 rl + 4 kq + i: row groups 4 hb + rl and 4 hb + rl + 2
                    float lo[4], hi[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        lo[i] = acc[4 * hb + rl][j][i];
                        hi[i] = acc[4 * hb + rl + 2][j][i];
                    }
                    const int jd0 = 16 * rl + 4 * kq;
                    if (is_q || is_k) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float2 cs = gld_f2(p.rope + (size_t)pos * 32 + jd0 + i);
                            const float x0 = lo[i] * cs.x - hi[i] * cs.y, x1 = lo[i] * cs.y + hi[i] * cs.x;
                            lo[i] = x0;
                            hi[i] = x1;
                        }
                    }
                    if (is_q) {
                        // query operands: (token group, head, d half), lane n + 16 (jd0 / 8), elements jd0 % 8 ..
                        const __amdgpu_buffer_rsrc_t qr = dev_rsrc(p.q, (uint32_t)(ntg * nq) * 4096u);
                        const uint32_t ln = (uint32_t)(n + 16 * (jd0 / 8)), e0 = (uint32_t)(jd0 % 8) * 2u;
                        u32x2v lh, ll, hh, hl;
                        split4(lo, lh, ll);
                        split4(hi, hh, hl);
                        const uint32_t u0 = (uint32_t)((tg * nq + head) * 2);
                        st8_dev(qr, ((u0 * 2u + 0u) * 64u + ln) * 16u + e0, lh);
                        st8_dev(qr, ((u0 * 2u + 1u) * 64u + ln) * 16u + e0, ll);
                        st8_dev(qr, (((u0 + 1u) * 2u + 0u) * 64u + ln) * 16u + e0, hh);
                        st8_dev(qr, (((u0 + 1u) * 2u + 1u) * 64u + ln) * 16u + e0, hl);
                    } else {
                        // K or V cache rows: layer l, KV head g, position pos, dimensions jd0 .. and jd0 + 32 ..
                        const int g = is_k ? head - nq : head - nq - nkv;
                        uint16_t* base = (is_k ? S.args.kc : S.args.vc) + (((size_t)l * nkv + g) * p.T.C + pos0) * 64;
                        const __amdgpu_buffer_rsrc_t cr = dev_rsrc(uni_ptr(base), (uint32_t)Tn * 128u);
                        const uint32_t off = (uint32_t)(tok * 64 + jd0) * 2u;
                        st8_dev(cr, off, u32x2v{(uint32_t)f2bf16(lo[0]) | ((uint32_t)f2bf16(lo[1]) << 16),
                                                (uint32_t)f2bf16(lo[2]) | ((uint32_t)f2bf16(lo[3]) << 16)});
                        st8_dev(cr, off + 64u, u32x2v{(uint32_t)f2bf16(hi[0]) | ((uint32_t)f2bf16(hi[1]) << 16),
                                                      (uint32_t)f2bf16(hi[2]) | ((uint32_t)f2bf16(hi[3]) << 16)});
                    }
                }
            }
        } else if constexpr (OPK == OP_PGU) {
            // m rows row0 + 16 rg + 4 kq + i (gate row groups rg < RG/2, up row groups rg + RG/2)
            const int nkm = p.T.f / 32;
            const __amdgpu_buffer_rsrc_t mr = dev_rsrc(pf_m(p), (uint32_t)(ntg * nkm) * 2048u);
#pragma unroll
            for (int rg = 0; rg < RG / 2; ++rg) {
                float m4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float gt = acc[rg][j][i], up = acc[rg + RG / 2][j][i];
                    m4[i] = gt / (1.0f + __expf(-gt)) * up;
                }
                const int mrow = (int)k.row0 + 16 * rg + 4 * kq;
                const uint32_t ln = (uint32_t)(n + 16 * ((mrow % 32) / 8)), e0 = (uint32_t)(mrow % 8) * 2u;
                u32x2v mh, ml;
                split4(m4, mh, ml);
                st8_dev(mr, pf_unit((uint32_t)tg, (uint32_t)nkm, (uint32_t)(mrow / 32), 0, ln) + e0, mh);
                st8_dev(mr, pf_unit((uint32_t)tg, (uint32_t)nkm, (uint32_t)(mrow / 32), 1, ln) + e0, ml);
            }
        } else {
            // O-projection / down: this K slice's partial rows of the prompt's tokens (the next RMSNorm
            // tasks add the slices to the residual)
            if (tok >= Tn) continue;
            const __amdgpu_buffer_rsrc_t pr =
                dev_rsrc(OPK == OP_POPROJ ? pf_po(p, k.part) : pf_pd(p, k.part), (uint32_t)(pf_rows(p) * 4));
#pragma unroll
            for (int rg = 0; rg < RG; ++rg)
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(u32x4, acc[rg][j]), pr,
                    (uint32_t)((size_t)tok * h + k.row0 + 16 * rg + 4 * kq) * 4u, 0, 16);
        }
    }
    return true;
}

// Causal attention of the 16 query tokens 16 qg .. of one KV group (head_dim 64): compute
// wave w takes the group's query heads w, w + 4, ...  For each block of 16 keys (cache
// slots 0 .. the group's last query position), the scores S^T = K Q^T come from the
// matrix cores (keys as rows, the 16 tokens as columns; the query in two bf16 parts),
// the softmax runs online per column, and O^T += V^T P^T on the matrix cores (P in two
// parts), as in the decode attention's layout.  The result goes to the O-projection's
// operands (two parts).  K/V rows of the prompt were written by this launch's QKV tiles.
__device__ __noinline__ bool op_pattn(const Params* pp, uint32_t slot_, uint32_t page0, uint32_t t_, uint32_t epoch_) {
    constexpr int D = 64;
    const Task k = fifo_task(slot_);
    Ctx c = make_ctx(t_, epoch_);
    CParams& p = P(pp);
    (void)page0;
    const int lane = c.lane, wave = c.wave, n = lane % 16, kq = lane / 16;
    const int l = k.layer, g = k.part, qg = (int)k.seq, G = p.T.grp, nq = p.T.nq, nkv = p.T.nkv, Tn = p.T.pf_T;
    const int ntg = pf_ntg(p);
    const int32_t pos0 = (int32_t)uni((uint32_t)S.args.pos0);
    if (!await_inputs(pp, k, c)) return false;
    tmark(c, 0);
    const int32_t kmax = pos0 + min(16 * qg + 15, Tn - 1);  // the last key any query of the group sees
    const int nblk = kmax / 16 + 1;
    const int32_t qpos = pos0 + 16 * qg + n;  // this lane's query position
    const size_t row0 = ((size_t)l * nkv + g) * (size_t)p.T.C;
    const __amdgpu_buffer_rsrc_t kr = dev_rsrc(uni_ptr(S.args.kc) + row0 * D, (uint32_t)(kmax + 1) * D * 2u);
    const __amdgpu_buffer_rsrc_t vr = dev_rsrc(uni_ptr(S.args.vc) + row0 * D, (uint32_t)(kmax + 1) * D * 2u);
    const __amdgpu_buffer_rsrc_t qr = dev_rsrc(p.q, (uint32_t)(ntg * nq) * 4096u);
    const int nko = nq * D / 32;
    const __amdgpu_buffer_rsrc_t orr = dev_rsrc(pf_o(p), (uint32_t)(ntg * nko) * 2048u);
    const float scale = 0.125f;  // 1 / sqrt(64)
    for (int hh = wave; hh < G; hh += NCW) {
        const int head = g * G + hh;
        u32x4v qb[2][NPART];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int pt = 0; pt < NPART; ++pt)
                qb[ks][pt] = __builtin_bit_cast(
                    u32x4v, __builtin_amdgcn_raw_buffer_load_b128(
                                qr, ((((uint32_t)(qg * nq + head) * 2u + ks) * 2u + pt) * 64u + lane) * 16u, 0, 16));
        f32x4v oacc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) oacc[t] = f32x4v{0.f, 0.f, 0.f, 0.f};
        float M = -INFINITY, Lp = 0.f;
        // K rows 16 kb + n (A operand: dimensions 32 ks + 8 kq ..), V words of keys 16 kb + 4 kq + jj,
        // dimensions 4 n .. 4 n + 3; rows past kmax are read as row kmax (masked below).  The next key
        // block's loads are issued before the current one's products.
        auto load_kv = [&](int kb, u32x4v (&ka)[2], u32x2v (&vw)[4]) {
            const uint32_t krow = (uint32_t)min(16 * kb + n, kmax);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                ka[ks] = __builtin_bit_cast(
                    u32x4v, __builtin_amdgcn_raw_buffer_load_b128(kr, (krow * D + 32 * ks + 8 * kq) * 2u, 0, 16));
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const uint32_t vrow = (uint32_t)min(16 * kb + 4 * kq + jj, kmax);
                vw[jj] = __builtin_amdgcn_raw_buffer_load_b64(vr, (vrow * D + 4 * n) * 2u, 0, 16);
            }
        };
        u32x4v kan[2];
        u32x2v vwn[4];
        load_kv(0, kan, vwn);
        for (int kb = 0; kb < nblk; ++kb) {
            u32x4v ka[2] = {kan[0], kan[1]};
            u32x2v vw[4] = {vwn[0], vwn[1], vwn[2], vwn[3]};
            load_kv(kb + 1, kan, vwn);  // (unconditional: rows past kmax read row kmax, unused)
            f32x4v s = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int pt = 0; pt < NPART; ++pt)
                    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, ka[ks]),
                                                                __builtin_bit_cast(bf16x8v, qb[ks][pt]), s, 0, 0, 0);
            // this lane: keys 16 kb + 4 kq + i of query column n
            float sc[4], mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sc[i] = 16 * kb + 4 * kq + i <= qpos ? s[i] * scale : -INFINITY;
                mx = fmaxf(mx, sc[i]);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float mn = fmaxf(M, mx);
            const float mref = mn == -INFINITY ? 0.f : mn;
            const float corr = __expf(M - mref);
            Lp *= corr;
#pragma unroll
            for (int t = 0; t < 4; ++t) oacc[t] *= corr;
            M = mn;
            float pr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pr[i] = __expf(sc[i] - mref);
                Lp += pr[i];
            }
            u32x2v ph, pl;
            split4(pr, ph, pl);
            // A operand t: V^T, row n standing for dimension 4 n + t, keys 4 kq + jj
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int cw = t / 2;
                const uint32_t a01 = (t & 1) ? (vw[0][cw] >> 16) | (vw[1][cw] & 0xffff0000u)
                                             : (vw[0][cw] & 0xffffu) | (vw[1][cw] << 16);
                const uint32_t a23 = (t & 1) ? (vw[2][cw] >> 16) | (vw[3][cw] & 0xffff0000u)
                                             : (vw[2][cw] & 0xffffu) | (vw[3][cw] << 16);
                const s16x4v av = __builtin_bit_cast(s16x4v, u32x2v{a01, a23});
                oacc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, __builtin_bit_cast(s16x4v, ph), oacc[t], 0, 0, 0);
                oacc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, __builtin_bit_cast(s16x4v, pl), oacc[t], 0, 0, 0);
            }
        }
        if (hh == wave) tmark(c, 1);
        float Lt = Lp + __shfl_xor(Lp, 16, 64);
        Lt += __shfl_xor(Lt, 32, 64);
        const float inv = 1.0f / Lt;
        // O rows d = 16 kq + 4 r + t of column n: two 8-dimension chunks per lane
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            float o8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o8[e] = oacc[e % 4][2 * cc + e / 4] * inv;
            u32x4v hi, lo;
            split8(o8, hi, lo);
            const int col = head * D + 16 * kq + 8 * cc;
            const uint32_t ln = (uint32_t)(n + 16 * ((col % 32) / 8));
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, hi), orr,
                                                   pf_unit((uint32_t)qg, (uint32_t)nko, (uint32_t)(col / 32), 0, ln), 0, 16);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, lo), orr,
                                                   pf_unit((uint32_t)qg, (uint32_t)nko, (uint32_t)(col / 32), 1, ln), 0, 16);
        }
    }
    return true;
}

// LM-head tile for the last prompt token: the several-sequence GEMV with one column (the
// final normalised token, LM operands), then the logits and the tile's argmax (packed
// 64-bit atomic max, as the decode LM head).
template <int KT>
__device__ __noinline__ bool op_plm(const Params* pp, uint32_t slot_, uint32_t page0, uint32_t t_, uint32_t epoch_) {
    constexpr int NBW = KT / 128;
    page0 = uni(page0);
    const Task k = fifo_task(slot_);
    Ctx c = make_ctx(t_, epoch_);
    CParams& p = P(pp);
    const int lane = c.lane, wave = c.wave, tid = c.tid;
    if (!await_inputs(pp, k, c)) return false;
    const __amdgpu_buffer_rsrc_t r = dev_rsrc(pf_lm(p), (uint32_t)(KT / 32) * 2048u);
    u32x4v bo[NBW][NPART];
#pragma unroll
    for (int i = 0; i < NBW; ++i)
#pragma unroll
        for (int pt = 0; pt < NPART; ++pt)
            bo[i][pt] = __builtin_bit_cast(
                u32x4v, __builtin_amdgcn_raw_buffer_load_b128(
                            r, (((uint32_t)(4 * i + wave) * 2u + pt) * 64u + lane) * 16u, 0, 16));
    tmark(c, 0);
    const uint32_t nrg = k.wbytes / (KT * 2) / 16;
    if (!gemv_mfma_b<KT>(pp, wave, lane, page0, nrg, bo, 1, k.id)) return false;
    if (!cbarrier(pp, c, k.id)) return false;
    tmark(c, 1);
    float* logits = S.args.logits;
    float bv = -INFINITY;
    uint32_t bi = 0xffffffffu;
    for (int i = tid; i < (int)k.nrows; i += NCW * 64) {  // rows in increasing order per lane: the first maximum is kept
        const float v = tile_res(i, 0, 1);
        if (logits) gst(logits + k.row0 + i, v);
        if (v > bv) {
            bv = v;
            bi = k.row0 + (uint32_t)i;
        }
    }
    const uint32_t ub = __float_as_uint(bv);
    const uint32_t ord = (ub & 0x80000000u) ? ~ub : (ub | 0x80000000u);
    unsigned long long key = bi == 0xffffffffu ? 0ull : (((unsigned long long)ord << 32) | (0xffffffffu - bi));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const unsigned long long other = __shfl_xor(key, o, 64);
        key = other > key ? other : key;
    }
    if (lane == 0 && key)
        __hip_atomic_fetch_max((g_u64*)&p.key[c.parity * KEY_SLOTS * p.T.B], key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}
