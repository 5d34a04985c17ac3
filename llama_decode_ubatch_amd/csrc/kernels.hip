// gfx950 (CDNA4) kernels of the decode step.  Layout conventions are in
// kernels.h.  Every kernel checks its own bounds from its arguments; the
// launchers derive grids from the same arguments.
#include "kernels.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

namespace ubd {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------- conversions
__device__ __forceinline__ uint16_t f2bf(float f) {
    uint32_t b = __float_as_uint(f);
    b += 0x7FFFu + ((b >> 16) & 1u);   // round to nearest even
    return (uint16_t)(b >> 16);
}
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ float h2f(uint16_t h) {
    _Float16 v;
    __builtin_memcpy(&v, &h, 2);
    return (float)v;
}
__device__ __forceinline__ uint16_t f2h(float f) {
    _Float16 v = (_Float16)f;          // IEEE round to nearest even
    uint16_t h;
    __builtin_memcpy(&h, &v, 2);
    return h;
}

__device__ __forceinline__ void store_act(const Act &o, size_t idx, float v) {
    if (o.f32) {
        o.f32[idx] = v;
    } else {
        uint16_t h = f2bf(v);
        o.hi[idx] = h;
        o.lo[idx] = f2bf(v - bf2f(h));
    }
}

template <typename T>
__device__ __forceinline__ T ldg_nt(const T *p) {
    return __builtin_nontemporal_load(p);
}

// --------------------------------------------------------------- matvec
// "Skinny" product y[t][n] = sum_k W[n][k] x[t][k] for up to 16 tokens per
// block of grid.y, on the matrix cores: A = a 16-row weight tile straight
// from HBM (already in fragment order), B = the activations of 16 tokens.
// MFMA output layout: lane l holds rows 4*(l/16)+i (i = 0..3) of the 16-row
// block for token l%16.  The k-steps are split over NW waves and reduced
// through LDS; wave 0 runs the epilogue.
template <int WT> struct WT_;
template <> struct WT_<W_F32> { static constexpr int KSTEP = 16, U = 8; };
template <> struct WT_<W_BF16> { static constexpr int KSTEP = 32, U = 8; };
template <> struct WT_<W_Q8> { static constexpr int KSTEP = 64, U = 4; };

__device__ __forceinline__ bf16x8_t i8x8_to_bf16(uint32_t w0, uint32_t w1) {
    // |code| <= 127 has at most 7 significant bits: exact in bf16, so the
    // top half of the f32 value is the bf16 value.
    u16x8_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[i] = (uint16_t)(__float_as_uint((float)(int8_t)(w0 >> (8 * i))) >> 16);
        r[4 + i] = (uint16_t)(__float_as_uint((float)(int8_t)(w1 >> (8 * i))) >> 16);
    }
    return __builtin_bit_cast(bf16x8_t, r);
}

template <int WT, int RB>
struct StepIn {
    u32x4_t w[RB];
    u32x4_t xh, xl, xh2, xl2;          // bf16: xh/xl; q8: block 0 (xh, xl), block 1 (xh2, xl2); f32: xh
    u32x2_t sc[RB][2];                  // q8 scales of rows 4g..4g+3, blocks 2s, 2s+1
};

template <int WT, int RB>
__device__ __forceinline__ void load_step(const LinearArgs &a, int rb0, int s, int steps,
                                          int lane, int tok, bool tok_ok, StepIn<WT, RB> &in) {
    const int g = lane >> 4;
#pragma unroll
    for (int j = 0; j < RB; ++j) {
        const size_t tile = (size_t)(rb0 + j) * steps + s;
        in.w[j] = ldg_nt((const u32x4_t *)((const char *)a.w + tile * 1024 + lane * 16));
    }
    if (WT == W_F32) {
        in.xh = tok_ok ? *(const u32x4_t *)(a.x.f32 + (size_t)tok * a.x.ld + 16 * s + 4 * g)
                       : u32x4_t{0, 0, 0, 0};
    } else if (WT == W_BF16) {
        const size_t o = (size_t)tok * a.x.ld + 32 * s + 8 * g;
        in.xh = tok_ok ? *(const u32x4_t *)(a.x.hi + o) : u32x4_t{0, 0, 0, 0};
        in.xl = tok_ok ? *(const u32x4_t *)(a.x.lo + o) : u32x4_t{0, 0, 0, 0};
    } else {
        const size_t o = (size_t)tok * a.x.ld + 64 * s + 8 * g;
        in.xh = tok_ok ? *(const u32x4_t *)(a.x.hi + o) : u32x4_t{0, 0, 0, 0};
        in.xl = tok_ok ? *(const u32x4_t *)(a.x.lo + o) : u32x4_t{0, 0, 0, 0};
        in.xh2 = tok_ok ? *(const u32x4_t *)(a.x.hi + o + 32) : u32x4_t{0, 0, 0, 0};
        in.xl2 = tok_ok ? *(const u32x4_t *)(a.x.lo + o + 32) : u32x4_t{0, 0, 0, 0};
        const int KB = a.K / 32;
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            const size_t b0 = ((size_t)(rb0 + j) * KB + 2 * s) * 16 + 4 * g;
            in.sc[j][0] = *(const u32x2_t *)(a.wscale + b0);
            in.sc[j][1] = *(const u32x2_t *)(a.wscale + b0 + 16);
        }
    }
}

template <int WT, int RB>
__device__ __forceinline__ void mfma_step(const StepIn<WT, RB> &in, f32x4_t *acc) {
    if (WT == W_F32) {
#pragma unroll
        for (int j = 0; j < RB; ++j) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(in.w[j][e]),
                                                              __uint_as_float(in.xh[e]), acc[j], 0, 0, 0);
        }
    } else if (WT == W_BF16) {
        const bf16x8_t xh = __builtin_bit_cast(bf16x8_t, in.xh);
        const bf16x8_t xl = __builtin_bit_cast(bf16x8_t, in.xl);
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            const bf16x8_t A = __builtin_bit_cast(bf16x8_t, in.w[j]);
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, xh, acc[j], 0, 0, 0);
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, xl, acc[j], 0, 0, 0);
        }
    } else {
        const bf16x8_t xh0 = __builtin_bit_cast(bf16x8_t, in.xh);
        const bf16x8_t xl0 = __builtin_bit_cast(bf16x8_t, in.xl);
        const bf16x8_t xh1 = __builtin_bit_cast(bf16x8_t, in.xh2);
        const bf16x8_t xl1 = __builtin_bit_cast(bf16x8_t, in.xl2);
        const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            const bf16x8_t A0 = i8x8_to_bf16(in.w[j][0], in.w[j][1]);
            const bf16x8_t A1 = i8x8_to_bf16(in.w[j][2], in.w[j][3]);
            f32x4_t d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, xh0, z, 0, 0, 0);
            d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, xl0, d0, 0, 0, 0);
            f32x4_t d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, xh1, z, 0, 0, 0);
            d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, xl1, d1, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t s0w = in.sc[j][0][i >> 1], s1w = in.sc[j][1][i >> 1];
                const float s0 = h2f((uint16_t)(s0w >> (16 * (i & 1))));
                const float s1 = h2f((uint16_t)(s1w >> (16 * (i & 1))));
                acc[j][i] += s0 * d0[i] + s1 * d1[i];
            }
        }
    }
}

__device__ __forceinline__ void store4(float *p, f32x4_t v) { *(f32x4_t *)p = v; }

// Epilogue of one MFMA output fragment: token t and four consecutive output
// rows n..n+3 (for SWIGLU: gate values v, up values u, output columns
// n..n+3).  ATOMIC accumulates a split-K partial into the residual.
template <int EPI, bool ATOMIC>
__device__ __forceinline__ void epilogue4(const LinearArgs &a, int t, int n, f32x4_t v, f32x4_t u) {
    if (EPI == EPI_STORE || EPI == EPI_RESID) {
        float *p = a.y + (size_t)t * a.ldy + n;
        if (EPI == EPI_RESID && ATOMIC) {
#pragma unroll
            for (int i = 0; i < 4; ++i) atomicAdd(p + i, v[i]);
        } else if (EPI == EPI_RESID) {
            f32x4_t o = *(f32x4_t *)p;
            store4(p, o + v);
        } else {
            store4(p, v);
        }
    } else if (EPI == EPI_LOGITS) {
        const int row = a.row_map[t];
        store4(a.logits + (size_t)row * a.N + n, v);
    } else if (EPI == EPI_SWIGLU) {
        const size_t o = (size_t)t * a.out.ld + n;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float gt = v[i], up = u[i];
            store_act(a.out, o + i, gt / (1.0f + expf(-gt)) * up);
        }
    } else if (EPI == EPI_QKV) {
        const QKVEpi &q = a.qkv;
        const int hd = q.head_dim;
        if (n < q.n_q_rows + q.n_k_rows) {
            const int pos = a.tok.pos[t];
            const int base = n < q.n_q_rows ? 0 : q.n_q_rows;
            const int d = (n - base) % hd;
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
                const double ang = (double)pos * q.inv_freq[(d >> 1) + pr];
                double sn, cs;
                sincos(ang, &sn, &cs);
                const float c = (float)cs, sf = (float)sn;
                const float x0 = v[2 * pr], x1 = v[2 * pr + 1];
                v[2 * pr] = x0 * c - x1 * sf;
                v[2 * pr + 1] = x0 * sf + x1 * c;
            }
        }
        if (n < q.n_q_rows) {
            store4(q.q_out + (size_t)t * q.n_q_rows + n, v);
        } else if (n < q.n_q_rows + q.n_k_rows) {
            const int o = n - q.n_q_rows, head = o / hd, d = o % hd;
            const size_t idx = (((size_t)a.tok.stream[t] * q.n_head_kv + head) * q.n_cells + a.tok.cell[t]) * hd + d;
            if (q.type_k == KV_F32) {
                store4((float *)q.k_cache + idx, v);
            } else {
                u16x4_t h = {f2h(v[0]), f2h(v[1]), f2h(v[2]), f2h(v[3])};
                *(u16x4_t *)((uint16_t *)q.k_cache + idx) = h;
            }
        } else {
            const int o = n - q.n_q_rows - q.n_k_rows, head = o / hd, d = o % hd;
            const size_t base = ((size_t)a.tok.stream[t] * q.n_head_kv + head) * hd + d;
            const int cell = a.tok.cell[t];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const size_t idx = (base + i) * q.n_cells + cell;
                if (q.type_v == KV_F32)
                    ((float *)q.v_cache)[idx] = v[i];
                else
                    ((uint16_t *)q.v_cache)[idx] = f2h(v[i]);
            }
        }
    }
}

template <int WT, int EPI, int NW>
__global__ __launch_bounds__(64 * NW) void linear_small_kernel(LinearArgs a) {
    constexpr int RB = EPI == EPI_SWIGLU ? 2 : 1;
    constexpr int KSTEP = WT_<WT>::KSTEP, U = WT_<WT>::U;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int rb0 = blockIdx.x * RB;
    const int t0 = blockIdx.y * 16;
    const int n_tok = min(16, a.T - t0);
    const bool tok_ok = r < n_tok;
    const int tok = t0 + (tok_ok ? r : 0);
    const int steps = a.K / KSTEP;
    const int s0 = wave * steps / NW, s1 = (wave + 1) * steps / NW;

    f32x4_t acc[RB];
#pragma unroll
    for (int j = 0; j < RB; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    int s = s0;
    for (; s + U <= s1; s += U) {
        StepIn<WT, RB> in[U];
#pragma unroll
        for (int u = 0; u < U; ++u) load_step<WT, RB>(a, rb0, s + u, steps, lane, tok, tok_ok, in[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) mfma_step<WT, RB>(in[u], acc);
    }
    for (; s < s1; ++s) {
        StepIn<WT, RB> in;
        load_step<WT, RB>(a, rb0, s, steps, lane, tok, tok_ok, in);
        mfma_step<WT, RB>(in, acc);
    }

    if (NW > 1) {
        __shared__ f32x4_t red[NW > 1 ? NW - 1 : 1][RB][64];
        if (wave > 0) {
#pragma unroll
            for (int j = 0; j < RB; ++j) red[wave - 1][j][lane] = acc[j];
        }
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int w = 0; w < NW - 1; ++w)
#pragma unroll
            for (int j = 0; j < RB; ++j) acc[j] += red[w][j][lane];
    }
    if (!tok_ok) return;
    const int t = t0 + r;
    if (EPI == EPI_SWIGLU)
        epilogue4<EPI, false>(a, t, blockIdx.x * 16 + 4 * g, acc[0], acc[RB - 1]);
    else
        epilogue4<EPI, false>(a, t, rb0 * 16 + 4 * g, acc[0], acc[0]);
}

// ----------------------------------------------------------------- GEMM
// Product for bf16 / q8_0 weights and many tokens (prefill).  Work-group
// tile: 256 weight rows (4 waves x 4 row blocks of 16) x BT tokens; k
// advances 64 values per stage.  A (weights) is read straight from HBM in
// fragment order; B (the hi plane of the activations) goes through LDS in
// fragment order, with the next stage prefetched into registers.  Tiles are
// numbered so that the work-groups sharing a weight tile (all token tiles
// and k-splits) run on the same XCD and reuse it from that XCD's L2.
__device__ __forceinline__ bf16x8_t i8x8_scaled_bf16(uint32_t w0, uint32_t w1, float sc) {
    u16x8_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[i] = f2bf((float)(int8_t)(w0 >> (8 * i)) * sc);
        r[4 + i] = f2bf((float)(int8_t)(w1 >> (8 * i)) * sc);
    }
    return __builtin_bit_cast(bf16x8_t, r);
}

template <int WT, int EPI, int BT, int SPLITK>
__global__ __launch_bounds__(256) void gemm_kernel(LinearArgs a, int n_wtiles, int n_ttiles) {
    // q8_0: the codes enter the MFMA exactly (|code| <= 127 is exact in
    // bf16), the activations as hi + lo planes, and each 32-value block's
    // f16 scale multiplies that block's MFMA result, so only the f32
    // accumulation rounds.  bf16 weights use the hi plane only.
    constexpr bool Q8 = WT == W_Q8;
    constexpr int TB = BT / 16;
    constexpr int XCH = BT * 8 / 256;       // 16-byte activation chunks per thread per stage
    constexpr int XS = TB * 2 * 64;         // one plane: [token block][k half][lane]
    __shared__ u32x4_t xs[(Q8 ? 2 : 1) * XS];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int total = n_wtiles * n_ttiles * SPLITK;
    const int b = blockIdx.x;
    const int tile = (total % 8 == 0) ? (b % 8) * (total / 8) + b / 8 : b;
    const int ks = tile % SPLITK;
    const int tt = (tile / SPLITK) % n_ttiles;
    const int nt = tile / (SPLITK * n_ttiles);
    const int nrb = a.N / 16;
    const int rb0 = nt * 16 + wave * 4;
    const int t0 = tt * BT;
    const int nstage = a.K / 64;
    const int st0 = ks * nstage / SPLITK, st1 = (ks + 1) * nstage / SPLITK;
    const int steps = a.K / (WT == W_BF16 ? 32 : 64);
    const int KB = a.K / 32;
    const u32x4_t z4 = {0u, 0u, 0u, 0u};

    f32x4_t acc[4][TB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < TB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t xr[XCH], xrl[Q8 ? XCH : 1];
    u32x4_t wr[4][2];
    u32x2_t sc[4][2];

    auto load_stage = [&](int st) {
#pragma unroll
        for (int q = 0; q < XCH; ++q) {
            const int c = threadIdx.x + 256 * q;
            const int row = c >> 3, ch = c & 7;
            const int t = t0 + row;
            const size_t o = (size_t)t * a.x.ld + st * 64 + ch * 8;
            xr[q] = t < a.T ? *(const u32x4_t *)(a.x.hi + o) : z4;
            if (Q8) xrl[q] = t < a.T ? *(const u32x4_t *)(a.x.lo + o) : z4;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rb = rb0 + i;
            if (rb < nrb) {
                if (!Q8) {
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        wr[i][j] = ldg_nt((const u32x4_t *)((const char *)a.w +
                                                           ((size_t)rb * steps + 2 * st + j) * 1024 + lane * 16));
                } else {
                    wr[i][0] = ldg_nt((const u32x4_t *)((const char *)a.w + ((size_t)rb * steps + st) * 1024 +
                                                       lane * 16));
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        sc[i][j] = *(const u32x2_t *)(a.wscale + ((size_t)rb * KB + 2 * st + j) * 16 + 4 * g);
                }
            } else {
                wr[i][0] = wr[i][1] = z4;
                sc[i][0] = sc[i][1] = u32x2_t{0u, 0u};
            }
        }
    };

    if (st0 < st1) load_stage(st0);
    for (int st = st0; st < st1; ++st) {
        __syncthreads();
#pragma unroll
        for (int q = 0; q < XCH; ++q) {
            const int c = threadIdx.x + 256 * q;
            const int row = c >> 3, ch = c & 7;
            const int idx = ((row >> 4) * 2 + (ch >> 2)) * 64 + (ch & 3) * 16 + (row & 15);
            xs[idx] = xr[q];
            if (Q8) xs[XS + idx] = xrl[q];
        }
        __syncthreads();
        bf16x8_t A[4][2];
        f32x4_t S[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (!Q8) {
                A[i][0] = __builtin_bit_cast(bf16x8_t, wr[i][0]);
                A[i][1] = __builtin_bit_cast(bf16x8_t, wr[i][1]);
            } else {
                A[i][0] = i8x8_to_bf16(wr[i][0][0], wr[i][0][1]);
                A[i][1] = i8x8_to_bf16(wr[i][0][2], wr[i][0][3]);
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        S[i][j][e] = h2f((uint16_t)(sc[i][j][e >> 1] >> (16 * (e & 1))));
            }
        }
        if (st + 1 < st1) load_stage(st + 1);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            bf16x8_t B[TB];
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) B[tb] = __builtin_bit_cast(bf16x8_t, xs[(tb * 2 + j) * 64 + lane]);
            if (!Q8) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int tb = 0; tb < TB; ++tb)
                        acc[i][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[i][j], B[tb], acc[i][tb], 0, 0, 0);
            } else {
                const f32x4_t zf = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const bf16x8_t Bl = __builtin_bit_cast(bf16x8_t, xs[XS + (tb * 2 + j) * 64 + lane]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        f32x4_t d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[i][j], B[tb], zf, 0, 0, 0);
                        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[i][j], Bl, d, 0, 0, 0);
                        acc[i][tb] += S[i][j] * d;
                    }
                }
            }
        }
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rb = rb0 + i;
        if (rb >= nrb) continue;
        if (EPI == EPI_SWIGLU && (i & 1)) continue;
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const int t = t0 + tb * 16 + r;
            if (t >= a.T) continue;
            if (EPI == EPI_SWIGLU)
                epilogue4<EPI, false>(a, t, (rb >> 1) * 16 + 4 * g, acc[i][tb], acc[i + 1][tb]);
            else
                epilogue4<EPI, (SPLITK > 1)>(a, t, rb * 16 + 4 * g, acc[i][tb], acc[i][tb]);
        }
    }
}

template <int WT, int EPI, int BT, int SPLITK>
static void launch_gemm(const LinearArgs &a, hipStream_t s) {
    const int n_wtiles = (a.N + 255) / 256;
    const int n_ttiles = (a.T + BT - 1) / BT;
    const int total = n_wtiles * n_ttiles * SPLITK;
    hipLaunchKernelGGL((gemm_kernel<WT, EPI, BT, SPLITK>), dim3(total), dim3(256), 0, s, a, n_wtiles, n_ttiles);
}

// True if the product was issued as a GEMM (bf16 / q8_0 weights, >= 64
// tokens, K a multiple of 64).
template <int WT, int EPI>
static bool try_gemm(const LinearArgs &a, hipStream_t s) {
    if constexpr (WT == W_F32) {
        return false;
    } else {
    if (a.T < 64 || a.K % 64) return false;
    if (EPI == EPI_SWIGLU && a.N % 32) return false;
    const int n_wtiles = (a.N + 255) / 256;
    const bool big = (long)n_wtiles * ((a.T + 127) / 128) >= 256;
    if (EPI == EPI_RESID) {
        const long tiles = (long)n_wtiles * ((a.T + 63) / 64);
        if (tiles >= 256 || a.K < 256) {
            launch_gemm<WT, EPI, 64, 1>(a, s);
        } else if (tiles * 2 >= 256 || a.K < 512) {
            launch_gemm<WT, EPI, 64, 2>(a, s);
        } else {
            launch_gemm<WT, EPI, 64, 4>(a, s);
        }
        return true;
    }
    if (big && WT != W_Q8)
        launch_gemm<WT, EPI, 128, 1>(a, s);
    else
        launch_gemm<WT, EPI, 64, 1>(a, s);
    return true;
    }
}

template <int WT, int EPI>
static void launch_linear_wt_epi(const LinearArgs &a, hipStream_t s) {
    constexpr int RB = EPI == EPI_SWIGLU ? 2 : 1;
    if (try_gemm<WT, EPI>(a, s)) return;
    dim3 grid(a.N / 16 / RB, (a.T + 15) / 16);
    const long blocks = (long)grid.x * grid.y;
    if (blocks >= 2048)
        hipLaunchKernelGGL((linear_small_kernel<WT, EPI, 4>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((linear_small_kernel<WT, EPI, 8>), grid, dim3(512), 0, s, a);
}

template <int WT>
static void launch_linear_wt(const LinearArgs &a, hipStream_t s) {
    switch (a.epi) {
    case EPI_STORE: launch_linear_wt_epi<WT, EPI_STORE>(a, s); break;
    case EPI_RESID: launch_linear_wt_epi<WT, EPI_RESID>(a, s); break;
    case EPI_SWIGLU: launch_linear_wt_epi<WT, EPI_SWIGLU>(a, s); break;
    case EPI_QKV: launch_linear_wt_epi<WT, EPI_QKV>(a, s); break;
    case EPI_LOGITS: launch_linear_wt_epi<WT, EPI_LOGITS>(a, s); break;
    }
}

void launch_linear(const LinearArgs &a, hipStream_t s) {
    if (a.T <= 0 || a.N <= 0) return;
    switch (a.wtype) {
    case W_F32: launch_linear_wt<W_F32>(a, s); break;
    case W_BF16: launch_linear_wt<W_BF16>(a, s); break;
    case W_Q8: launch_linear_wt<W_Q8>(a, s); break;
    }
}

// ------------------------------------------------------------ embedding
__global__ __launch_bounds__(256) void embed_kernel(int wtype, const void *table, const uint16_t *scales,
                                                    int d, TokInfo ti, float *x, int32_t *cell_pos,
                                                    int32_t *cell_seq, int n_cells) {
    const int t = blockIdx.x;
    const size_t row = (size_t)ti.token[t];
    float *xo = x + (size_t)t * d;
    for (int j = threadIdx.x; j < d; j += blockDim.x) {
        float v;
        if (wtype == W_F32)
            v = ((const float *)table)[row * d + j];
        else if (wtype == W_BF16)
            v = bf2f(((const uint16_t *)table)[row * d + j]);
        else
            v = (float)((const int8_t *)table)[row * d + j] * h2f(scales[row * (d / 32) + j / 32]);
        xo[j] = v;
    }
    if (threadIdx.x == 0) {
        const size_t c = (size_t)ti.stream[t] * n_cells + ti.cell[t];
        cell_pos[c] = ti.pos[t];
        cell_seq[c] = ti.seq[t];
    }
}

void launch_embed(int wtype, const void *table, const uint16_t *scales, int d, const TokInfo &ti, int T,
                  float *x, int32_t *cell_pos, int32_t *cell_seq, int n_cells, hipStream_t s) {
    if (T <= 0) return;
    hipLaunchKernelGGL(embed_kernel, dim3(T), dim3(256), 0, s, wtype, table, scales, d, ti, x, cell_pos,
                       cell_seq, n_cells);
}

// -------------------------------------------------------------- RMSNorm
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__global__ __launch_bounds__(256) void rmsnorm_kernel(const float *x, int ldx, const int32_t *row_map,
                                                      const float *gain, int d, float eps, Act out) {
    const int r = blockIdx.x;
    const int src = row_map ? row_map[r] : r;
    const float *xr = x + (size_t)src * ldx;
    float ss = 0.f;
    for (int j = threadIdx.x; j < d; j += blockDim.x) ss += xr[j] * xr[j];
    __shared__ float part[4];
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = part[0] + part[1] + part[2] + part[3];
    const float inv = 1.0f / sqrtf(tot / (float)d + eps);
    for (int j = threadIdx.x; j < d; j += blockDim.x)
        store_act(out, (size_t)r * out.ld + j, xr[j] * inv * gain[j]);
}

void launch_rmsnorm(const float *x, int ldx, const int32_t *row_map, int rows, const float *gain, int d,
                    float eps, const Act &out, hipStream_t s) {
    if (rows <= 0) return;
    hipLaunchKernelGGL(rmsnorm_kernel, dim3(rows), dim3(256), 0, s, x, ldx, row_map, gain, d, eps, out);
}

// ------------------------------------------------------------ attention
// Split-K attention over KV cells in f32 arithmetic (every config).
// Work item = (cell chunk, query tile, KV head).  A query tile is a run of
// ubatch tokens of one KV stream; its rows are (token, query head of the
// group).  Per 32/64-cell sub-tile: K (transposed) and V^T go to LDS, scores
// are masked by cell position / sequence, an online softmax keeps (m, l),
// and P*V accumulates.  The chunk's (m, l, O) are combined later.
template <int HD> struct AttnCfg {
    static constexpr int ROWS = HD >= 128 ? 32 : 64;
    static constexpr int SUB = HD >= 64 ? 32 : 64;
    static constexpr int NACC = (ROWS * HD + 255) / 256;
};

__device__ __forceinline__ float load_kv(const void *p, int type, size_t idx) {
    return type == KV_F32 ? ((const float *)p)[idx] : h2f(((const uint16_t *)p)[idx]);
}

template <int HD>
__global__ __launch_bounds__(256) void attn_partial_kernel(AttnArgs a) {
    using C = AttnCfg<HD>;
    constexpr int SUB = C::SUB, ROWS = C::ROWS;
    const int chunk = blockIdx.x, tile = blockIdx.y, g = blockIdx.z;
    const int t0 = a.tok.tiles[tile * 4 + 0], nt = a.tok.tiles[tile * 4 + 1];
    const int st = a.tok.tiles[tile * 4 + 2], nkv = a.tok.tiles[tile * 4 + 3];
    const int cbeg = chunk * ATTN_CHUNK;
    if (cbeg >= nkv) return;
    const int cend = min(nkv, cbeg + ATTN_CHUNK);
    const int G = a.n_head / a.n_head_kv;
    const int R = nt * G;
    const int tid = threadIdx.x;

    __shared__ float qs[ROWS][HD];
    __shared__ float Kt[HD][SUB + 1];
    __shared__ float Vt[HD][SUB + 1];
    __shared__ float ps[ROWS][SUB + 1];
    __shared__ int cpos[SUB], cseq[SUB];
    __shared__ float m_s[ROWS], l_s[ROWS], sc_s[ROWS];
    __shared__ int rpos[ROWS], rseq[ROWS];

    const float scale = 1.0f / sqrtf((float)HD);
    for (int e = tid; e < R * HD; e += 256) {
        const int row = e / HD, d = e % HD;
        const int t = t0 + row / G, h = g * G + row % G;
        qs[row][d] = a.q[(size_t)t * a.n_head * HD + h * HD + d] * scale;
    }
    if (tid < R) {
        const int t = t0 + tid / G;
        rpos[tid] = a.tok.pos[t];
        rseq[tid] = a.tok.seq[t];
        m_s[tid] = -INFINITY;
        l_s[tid] = 0.f;
    }
    float acc[C::NACC];
#pragma unroll
    for (int j = 0; j < C::NACC; ++j) acc[j] = 0.f;

    const size_t kbase = ((size_t)st * a.n_head_kv + g) * a.n_cells * HD;  // [cell][hd]
    const size_t vbase = ((size_t)st * a.n_head_kv + g) * HD * a.n_cells;  // [hd][cell]
    const int32_t *cp = a.cell_pos + (size_t)st * a.n_cells;
    const int32_t *cs = a.cell_seq + (size_t)st * a.n_cells;

    for (int sub = cbeg; sub < cend; sub += SUB) {
        const int ns = min(SUB, cend - sub);
        __syncthreads();
        for (int e = tid; e < SUB * HD; e += 256) {
            const int c = e / HD, d = e % HD;
            Kt[d][c] = c < ns ? load_kv(a.k_cache, a.type_k, kbase + (size_t)(sub + c) * HD + d) : 0.f;
        }
        for (int e = tid; e < SUB * HD; e += 256) {
            const int d = e / SUB, c = e % SUB;
            Vt[d][c] = c < ns ? load_kv(a.v_cache, a.type_v, vbase + (size_t)d * a.n_cells + sub + c) : 0.f;
        }
        if (tid < SUB) {
            cpos[tid] = tid < ns ? cp[sub + tid] : -1;
            cseq[tid] = tid < ns ? cs[sub + tid] : -1;
        }
        __syncthreads();
        for (int e = tid; e < R * SUB; e += 256) {
            const int row = e / SUB, c = e % SUB;
            float sv = -INFINITY;
            if (c < ns && cseq[c] == rseq[row] && cpos[c] >= 0 && cpos[c] <= rpos[row]) {
                float dot = 0.f;
#pragma unroll 8
                for (int d = 0; d < HD; ++d) dot += qs[row][d] * Kt[d][c];
                sv = dot;
            }
            ps[row][c] = sv;
        }
        __syncthreads();
        if (tid < R) {
            const float m_old = m_s[tid];
            float mx = m_old;
            for (int c = 0; c < ns; ++c) mx = fmaxf(mx, ps[tid][c]);
            float l = l_s[tid], sc = 1.f;
            if (mx != -INFINITY) {
                sc = m_old == -INFINITY ? 0.f : expf(m_old - mx);
                l *= sc;
                for (int c = 0; c < ns; ++c) {
                    const float sv = ps[tid][c];
                    const float p = sv == -INFINITY ? 0.f : expf(sv - mx);
                    ps[tid][c] = p;
                    l += p;
                }
            } else {
                for (int c = 0; c < ns; ++c) ps[tid][c] = 0.f;
            }
            for (int c = ns; c < SUB; ++c) ps[tid][c] = 0.f;
            m_s[tid] = mx;
            l_s[tid] = l;
            sc_s[tid] = sc;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < C::NACC; ++j) {
            const int e = tid + 256 * j;
            if (e < R * HD) {
                const int row = e / HD, d = e % HD;
                float o = acc[j] * sc_s[row];
                for (int c = 0; c < ns; ++c) o += ps[row][c] * Vt[d][c];
                acc[j] = o;
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < C::NACC; ++j) {
        const int e = tid + 256 * j;
        if (e < R * HD) {
            const int row = e / HD, d = e % HD;
            const int t = t0 + row / G, h = g * G + row % G;
            a.part_o[(((size_t)t * a.n_head + h) * a.max_chunks + chunk) * HD + d] = acc[j];
        }
    }
    if (tid < R) {
        const int t = t0 + tid / G, h = g * G + tid % G;
        float *ml = a.part_ml + (((size_t)t * a.n_head + h) * a.max_chunks + chunk) * 2;
        ml[0] = m_s[tid];
        ml[1] = l_s[tid];
    }
}

template <int HD>
__global__ __launch_bounds__(128) void attn_combine_kernel(AttnArgs a) {
    const int t = blockIdx.x / a.n_head, h = blockIdx.x % a.n_head;
    const int tile = a.tok.tile_of[t];
    const int nkv = a.tok.tiles[tile * 4 + 3];
    const int nch = (nkv + ATTN_CHUNK - 1) / ATTN_CHUNK;
    const float *ml = a.part_ml + ((size_t)t * a.n_head + h) * a.max_chunks * 2;
    float M = -INFINITY;
    for (int c = 0; c < nch; ++c) M = fmaxf(M, ml[2 * c]);
    float L = 0.f;
    for (int c = 0; c < nch; ++c)
        if (ml[2 * c] != -INFINITY) L += ml[2 * c + 1] * expf(ml[2 * c] - M);
    const float invL = L > 0.f ? 1.0f / L : 0.f;
    for (int d = threadIdx.x; d < HD; d += blockDim.x) {
        float o = 0.f;
        for (int c = 0; c < nch; ++c)
            if (ml[2 * c] != -INFINITY)
                o += a.part_o[(((size_t)t * a.n_head + h) * a.max_chunks + c) * HD + d] * expf(ml[2 * c] - M);
        store_act(a.out, (size_t)t * a.out.ld + h * HD + d, o * invL);
    }
}

template <int HD>
static void launch_attention_hd(const AttnArgs &a, hipStream_t s) {
    dim3 grid(a.max_chunks, a.n_tiles, a.n_head_kv);
    hipLaunchKernelGGL(attn_partial_kernel<HD>, grid, dim3(256), 0, s, a);
    hipLaunchKernelGGL(attn_combine_kernel<HD>, dim3(a.T * a.n_head), dim3(128), 0, s, a);
}

void launch_attention(const AttnArgs &a, hipStream_t s) {
    if (a.T <= 0) return;
    switch (a.head_dim) {
    case 32: launch_attention_hd<32>(a, s); break;
    case 64: launch_attention_hd<64>(a, s); break;
    case 128: launch_attention_hd<128>(a, s); break;
    }
}

// MFMA attention for f16 K/V (decode and prefill).  One wave = one block of
// 16 query rows (row = token x query head of a KV group; a decode token
// gives n_gqa rows) against a range of cells.  Scores are computed as
// S^T = K Q^T (A = 16 cells x 32 dims of K straight from the cache, B = the
// rows' q as f16 hi + lo), so lane (row r, group g) holds S[r][cells 4g+i]
// of each 16-cell block.  Two blocks give exactly the P fragment of P*V for
// the cell order {4g..4g+3, 16+4g..16+4g+3}, which V^T [dim][cell] supplies
// as two contiguous 8-byte runs.  Online softmax per row; SPLIT writes the
// range's (m, l, O) for a combine pass, otherwise O / l is stored.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

template <int HD, bool SPLIT, int NC>
__global__ __launch_bounds__(64) void attn_mfma_kernel(AttnArgs a) {
    constexpr int KK = HD / 32, DB = HD / 16;
    const int lane = threadIdx.x, r = lane & 15, g = lane >> 4;
    const int chunk = blockIdx.x, blk = blockIdx.y, grp = blockIdx.z;
    const int t0 = a.tok.tiles[blk * 4 + 0], nt = a.tok.tiles[blk * 4 + 1];
    const int st = a.tok.tiles[blk * 4 + 2], nscan = a.tok.tiles[blk * 4 + 3];
    const int G = a.n_head / a.n_head_kv;
    const int R = nt * G;
    int cbeg = 0, cend = nscan;
    if (SPLIT) {
        cbeg = chunk * NC;
        if (cbeg >= nscan) return;
        cend = min(nscan, cbeg + NC);
    }
    const float scale = 1.0f / sqrtf((float)HD);
    // this lane's query row (S^T layout: row = r)
    const bool row_ok = r < R;
    const int rt = t0 + (row_ok ? r / G : 0), rh = grp * G + (row_ok ? r % G : 0);
    const int rpos = a.tok.pos[rt], rseq = a.tok.seq[rt];
    f16x8_t qh[KK], ql[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float v = row_ok ? a.q[(size_t)rt * a.n_head * HD + rh * HD + 32 * kk + 8 * g + e] * scale : 0.f;
            const _Float16 h = (_Float16)v;
            qh[kk][e] = h;
            ql[kk][e] = (_Float16)(v - (float)h);
        }
    }
    const _Float16 *K = (const _Float16 *)a.k_cache + ((size_t)st * a.n_head_kv + grp) * a.n_cells * HD;
    const _Float16 *Vt = (const _Float16 *)a.v_cache + ((size_t)st * a.n_head_kv + grp) * HD * a.n_cells;
    const int32_t *cpos = a.cell_pos + (size_t)st * a.n_cells;
    const int32_t *cseq = a.cell_seq + (size_t)st * a.n_cells;

    float m = -INFINITY, l = 0.f;
    f32x4_t O[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) O[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int c0 = cbeg; c0 < cend; c0 += 32) {
        f32x4_t S[2];
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2) {
            const int cb = c0 + 16 * b2;
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const f16x8_t A = *(const f16x8_t *)(K + (size_t)(cb + r) * HD + 32 * kk + 8 * g);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qh[kk], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, ql[kk], acc, 0, 0, 0);
            }
            const int cc = cb + 4 * g;
            const int4 p4 = *(const int4 *)(cpos + cc);
            const int4 s4 = *(const int4 *)(cseq + cc);
            const int pp[4] = {p4.x, p4.y, p4.z, p4.w}, ss[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool vis = row_ok && cc + i < cend && ss[i] == rseq && pp[i] >= 0 && pp[i] <= rpos;
                acc[i] = vis ? acc[i] : -INFINITY;
            }
            S[b2] = acc;
        }
        float mx = fmaxf(fmaxf(fmaxf(S[0][0], S[0][1]), fmaxf(S[0][2], S[0][3])),
                         fmaxf(fmaxf(S[1][0], S[1][1]), fmaxf(S[1][2], S[1][3])));
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m, mx);
        const float alpha = (m_new == -INFINITY) ? 1.f : expf(m - m_new);
        float ps = 0.f;
        f16x8_t ph, pl;
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float sv = S[b2][i];
                const float p = sv == -INFINITY ? 0.f : expf(sv - m_new);
                ps += p;
                const _Float16 h = (_Float16)p;
                ph[4 * b2 + i] = h;
                pl[4 * b2 + i] = (_Float16)(p - (float)h);
            }
        ps += __shfl_xor(ps, 16, 64);
        ps += __shfl_xor(ps, 32, 64);
        l = l * alpha + ps;
        m = m_new;
        // O rows are 4g+i in this lane: fetch their rescale factors
        f32x4_t al;
#pragma unroll
        for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const _Float16 *vrow = Vt + (size_t)(16 * db + r) * a.n_cells;
            const f16x4_t v0 = *(const f16x4_t *)(vrow + c0 + 4 * g);
            const f16x4_t v1 = *(const f16x4_t *)(vrow + c0 + 16 + 4 * g);
            const f16x8_t B = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            f32x4_t o = O[db] * al;
            o = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph, B, o, 0, 0, 0);
            o = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl, B, o, 0, 0, 0);
            O[db] = o;
        }
    }
    // O: lane (dim r of each 16-dim block, group g) holds rows 4g+i
    f32x4_t lrow;
#pragma unroll
    for (int i = 0; i < 4; ++i) lrow[i] = __shfl(l, 4 * g + i, 64);
    if (SPLIT) {
        if (g == 0 && row_ok) {
            float *ml = a.part_ml + (((size_t)rt * a.n_head + rh) * a.max_chunks + chunk) * 2;
            ml[0] = m;
            ml[1] = l;
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 4 * g + i;
        if (row >= R) continue;
        const int t = t0 + row / G, h = grp * G + row % G;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int d = 16 * db + r;
            if (SPLIT)
                a.part_o[(((size_t)t * a.n_head + h) * a.max_chunks + chunk) * HD + d] = O[db][i];
            else
                store_act(a.out, (size_t)t * a.out.ld + h * HD + d, lrow[i] > 0.f ? O[db][i] / lrow[i] : 0.f);
        }
    }
}

template <int HD, int NC>
__global__ __launch_bounds__(128) void attn_combine_nc_kernel(AttnArgs a) {
    const int t = blockIdx.x / a.n_head, h = blockIdx.x % a.n_head;
    const int tile = a.tok.tile_of[t];
    const int nscan = a.tok.tiles[tile * 4 + 3];
    const int nch = (nscan + NC - 1) / NC;
    const float *ml = a.part_ml + ((size_t)t * a.n_head + h) * a.max_chunks * 2;
    float M = -INFINITY;
    for (int c = 0; c < nch; ++c) M = fmaxf(M, ml[2 * c]);
    float L = 0.f;
    for (int c = 0; c < nch; ++c)
        if (ml[2 * c] != -INFINITY) L += ml[2 * c + 1] * expf(ml[2 * c] - M);
    const float invL = L > 0.f ? 1.0f / L : 0.f;
    for (int d = threadIdx.x; d < HD; d += blockDim.x) {
        float o = 0.f;
        for (int c = 0; c < nch; ++c)
            if (ml[2 * c] != -INFINITY)
                o += a.part_o[(((size_t)t * a.n_head + h) * a.max_chunks + c) * HD + d] * expf(ml[2 * c] - M);
        store_act(a.out, (size_t)t * a.out.ld + h * HD + d, o * invL);
    }
}

template <int HD>
static void launch_attention_mfma_hd(const AttnArgs &a, hipStream_t s) {
    if (a.split) {
        dim3 grid(a.max_chunks, a.n_tiles, a.n_head_kv);
        hipLaunchKernelGGL((attn_mfma_kernel<HD, true, ATTN_DECODE_CHUNK>), grid, dim3(64), 0, s, a);
        hipLaunchKernelGGL((attn_combine_nc_kernel<HD, ATTN_DECODE_CHUNK>), dim3(a.T * a.n_head), dim3(128), 0, s,
                           a);
    } else {
        dim3 grid(1, a.n_tiles, a.n_head_kv);
        hipLaunchKernelGGL((attn_mfma_kernel<HD, false, ATTN_DECODE_CHUNK>), grid, dim3(64), 0, s, a);
    }
}

bool attn_mfma_ok(int type_k, int type_v, int head_dim, int n_gqa, int n_cells) {
    return type_k == KV_F16 && type_v == KV_F16 && n_gqa <= 16 && n_cells % 32 == 0 &&
           (head_dim == 32 || head_dim == 64 || head_dim == 128);
}

void launch_attention_mfma(const AttnArgs &a, hipStream_t s) {
    if (a.T <= 0) return;
    switch (a.head_dim) {
    case 32: launch_attention_mfma_hd<32>(a, s); break;
    case 64: launch_attention_mfma_hd<64>(a, s); break;
    case 128: launch_attention_mfma_hd<128>(a, s); break;
    }
}

int attn_tile_rows(int head_dim) { return head_dim >= 128 ? AttnCfg<128>::ROWS : AttnCfg<64>::ROWS; }

// --------------------------------------------------------------- argmax
__global__ __launch_bounds__(1024) void argmax_kernel(const float *logits, int ld, const int32_t *rows,
                                                      int n, int32_t *out) {
    const int r = blockIdx.x;
    const float *z = logits + (size_t)(rows ? rows[r] : r) * ld;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const float v = z[i];
        if (v > bv || (v == bv && i < bi)) {
            bv = v;
            bi = i;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (ov > bv || (ov == bv && oi < bi)) {
            bv = ov;
            bi = oi;
        }
    }
    __shared__ float sv[16];
    __shared__ int si[16];
    if ((threadIdx.x & 63) == 0) {
        sv[threadIdx.x >> 6] = bv;
        si[threadIdx.x >> 6] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < (int)(blockDim.x >> 6); ++w)
            if (sv[w] > bv || (sv[w] == bv && si[w] < bi)) {
                bv = sv[w];
                bi = si[w];
            }
        out[r] = bi == 0x7fffffff ? 0 : bi;
    }
}

void launch_argmax(const float *logits, int ld, const int32_t *rows, int n_rows, int n, int32_t *out,
                   hipStream_t s) {
    if (n_rows <= 0) return;
    hipLaunchKernelGGL(argmax_kernel, dim3(n_rows), dim3(1024), 0, s, logits, ld, rows, n, out);
}

// ------------------------------------------------------------- relayout
struct RelayoutArgs {
    RelayoutSrc src[3];
    int n_src, mode, K, N, steps, kstep, wtype;
    void *dst;
    uint16_t *dst_scales;
};

__device__ __forceinline__ void map_row(const RelayoutArgs &a, int row, int *si, int *sr) {
    if (a.mode == 1) {
        const int rb = row >> 4;
        *si = rb & 1;
        *sr = (rb >> 1) * 16 + (row & 15);
        return;
    }
    int r = row;
    for (int i = 0; i < a.n_src; ++i) {
        if (r < a.src[i].rows) {
            *si = i;
            *sr = r;
            return;
        }
        r -= a.src[i].rows;
    }
    *si = a.n_src - 1;
    *sr = r;
}

__global__ __launch_bounds__(256) void relayout_kernel(RelayoutArgs a) {
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t total = (size_t)(a.N / 16) * a.steps * 64;
    if (idx >= total) return;
    const size_t tile = idx >> 6;
    const int lane = (int)(idx & 63);
    const int rb = (int)(tile / a.steps), s = (int)(tile % a.steps);
    const int r = lane & 15, g = lane >> 4;
    int si, sr;
    map_row(a, rb * 16 + r, &si, &sr);
    char *dst = (char *)a.dst + idx * 16;
    if (a.wtype == W_F32) {
        const float *row = (const float *)a.src[si].data + (size_t)sr * a.K;
        *(u32x4_t *)dst = *(const u32x4_t *)(row + 16 * s + 4 * g);
    } else if (a.wtype == W_BF16) {
        const uint16_t *row = (const uint16_t *)a.src[si].data + (size_t)sr * a.K;
        *(u32x4_t *)dst = *(const u32x4_t *)(row + 32 * s + 8 * g);
    } else {
        const int8_t *row = (const int8_t *)a.src[si].data + (size_t)sr * a.K;
        *(u32x2_t *)dst = *(const u32x2_t *)(row + 64 * s + 8 * g);
        *(u32x2_t *)(dst + 8) = *(const u32x2_t *)(row + 64 * s + 32 + 8 * g);
    }
}

__global__ __launch_bounds__(256) void relayout_scales_kernel(RelayoutArgs a) {
    const int KB = a.K / 32;
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t total = (size_t)a.N * KB;
    if (idx >= total) return;
    const int r = (int)(idx & 15);
    const size_t rest = idx >> 4;
    const int b = (int)(rest % KB), rb = (int)(rest / KB);
    int si, sr;
    map_row(a, rb * 16 + r, &si, &sr);
    a.dst_scales[idx] = a.src[si].scales[(size_t)sr * KB + b];
}

void launch_relayout(int wtype, const RelayoutSrc *src, int n_src, int mode, int K, void *dst,
                     uint16_t *dst_scales, hipStream_t s) {
    RelayoutArgs a{};
    a.n_src = n_src;
    a.mode = mode;
    a.K = K;
    a.wtype = wtype;
    a.N = 0;
    for (int i = 0; i < n_src; ++i) {
        a.src[i] = src[i];
        a.N += src[i].rows;
    }
    a.kstep = wtype == W_F32 ? 16 : wtype == W_BF16 ? 32 : 64;
    a.steps = K / a.kstep;
    a.dst = dst;
    a.dst_scales = dst_scales;
    const size_t total = (size_t)(a.N / 16) * a.steps * 64;
    hipLaunchKernelGGL(relayout_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
    if (wtype == W_Q8) {
        const size_t ts = (size_t)a.N * (K / 32);
        hipLaunchKernelGGL(relayout_scales_kernel, dim3((unsigned)((ts + 255) / 256)), dim3(256), 0, s, a);
    }
}

// ---------------------------------------------------------- KV fill/read
// 64x64 tiles through LDS so that both the [n][Hk*hd] rows and the
// transposed V cache are touched in contiguous runs.
__global__ __launch_bounds__(256) void kv_store_kernel(const void *src, int src_type, int n,
                                                       const int32_t *cells, void *cache, int type,
                                                       int transposed, int stream, int n_head_kv, int hd,
                                                       int n_cells) {
    __shared__ float tileb[64][65];
    const int W = n_head_kv * hd;
    const int p0 = blockIdx.x * 64, j0 = blockIdx.y * 64;
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
        const int py = e / 64, jx = e % 64;
        const int p = p0 + py, j = j0 + jx;
        float v = 0.f;
        if (p < n && j < W) v = load_kv(src, src_type, (size_t)p * W + j);
        tileb[py][jx] = v;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
        int p, j;
        if (transposed) {
            j = j0 + e / 64;
            p = p0 + e % 64;
        } else {
            p = p0 + e / 64;
            j = j0 + e % 64;
        }
        if (p >= n || j >= W) continue;
        const float v = tileb[p - p0][j - j0];
        const int head = j / hd, d = j % hd;
        const size_t c = (size_t)cells[p];
        size_t idx;
        if (transposed)
            idx = (((size_t)stream * n_head_kv + head) * hd + d) * n_cells + c;
        else
            idx = (((size_t)stream * n_head_kv + head) * n_cells + c) * hd + d;
        if (type == KV_F32)
            ((float *)cache)[idx] = v;
        else
            ((uint16_t *)cache)[idx] = f2h(v);
    }
}

void launch_kv_store(const void *src, int src_type, int n, const int32_t *cells, void *cache, int type,
                     bool transposed, int stream, int n_head_kv, int hd, int n_cells, hipStream_t s) {
    if (n <= 0) return;
    const int W = n_head_kv * hd;
    dim3 grid((n + 63) / 64, (W + 63) / 64);
    hipLaunchKernelGGL(kv_store_kernel, grid, dim3(256), 0, s, src, src_type, n, cells, cache, type,
                       (int)transposed, stream, n_head_kv, hd, n_cells);
}

__global__ __launch_bounds__(256) void kv_load_kernel(const void *cache, int type, int transposed, int stream,
                                                      int cell0, int n, int n_head_kv, int hd, int n_cells,
                                                      float *out) {
    const int W = n_head_kv * hd;
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)n * W) return;
    const int p = (int)(idx / W), j = (int)(idx % W);
    const int head = j / hd, d = j % hd;
    const size_t c = (size_t)cell0 + p;
    size_t src;
    if (transposed)
        src = (((size_t)stream * n_head_kv + head) * hd + d) * n_cells + c;
    else
        src = (((size_t)stream * n_head_kv + head) * n_cells + c) * hd + d;
    out[idx] = load_kv(cache, type, src);
}

void launch_kv_load(const void *cache, int type, bool transposed, int stream, int cell0, int n, int n_head_kv,
                    int hd, int n_cells, float *out, hipStream_t s) {
    if (n <= 0) return;
    const size_t total = (size_t)n * n_head_kv * hd;
    hipLaunchKernelGGL(kv_load_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, cache, type,
                       (int)transposed, stream, cell0, n, n_head_kv, hd, n_cells, out);
}

}  // namespace ubd
