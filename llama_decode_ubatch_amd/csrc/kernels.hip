// gfx950 (CDNA4) kernels of the decode step.  Layout conventions are in
// kernels.h.  Every kernel checks its own bounds from its arguments; the
// launchers derive grids from the same arguments.
#include "kernels.h"

#include <type_traits>

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

namespace ubd {

Tuning g_tuning;
thread_local LaunchTiming g_launch_timing;

#define UBD_LAUNCH(K, G, B, SH, S, ...)                                                                         \
    do {                                                                                                        \
        if (g_launch_timing.stop) {                                                                             \
            hipExtLaunchKernelGGL(K, G, B, SH, S, g_launch_timing.start, g_launch_timing.stop, 0, __VA_ARGS__); \
            g_launch_timing.start = nullptr;                                                                    \
        } else {                                                                                                \
            hipLaunchKernelGGL(K, G, B, SH, S, __VA_ARGS__);                                                    \
        }                                                                                                       \
    } while (0)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------- conversions
__device__ __forceinline__ uint16_t f2bf(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);   // v_cvt_pk_bf16_f32: round to nearest even
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

// Activation planes of the LDS-staged decode products: value = hi + lo,
// bf16 planes for bf16 weights, f16 planes for q8_0 weights (whose codes
// enter f16 MFMAs).  The f16 planes hold |value| <= F16_PLANE_MAX; `big`
// records a value beyond it (the product then rescales its rows, see
// ldsx_rescale).
constexpr float F16_PLANE_MAX = 65504.f;
template <int WT>
__device__ __forceinline__ void split_hilo(float y, uint16_t &h, uint16_t &l, int &big) {
    if (WT == W_Q8) {
        big |= fabsf(y) > F16_PLANE_MAX;
        h = f2h(y);
        l = f2h(y - h2f(h));
    } else {
        h = f2bf(y);
        l = f2bf(y - bf2f(h));
    }
}

// Barrier that publishes the activation copy; for q8_0 it also tells every
// thread whether any thread saw a value beyond the f16 planes.
template <int WT>
__device__ __forceinline__ int copy_barrier(int big) {
    if (WT == W_Q8) return __syncthreads_or(big);
    __syncthreads();
    return 0;
}

// element index of activation (token t, value c) in either layout
__device__ __forceinline__ size_t act_idx(const Act &o, int t, int c) {
    if (!o.tiled) return (size_t)t * o.ld + c;
    return ((size_t)(t >> 4) * (o.ld >> 5) + (c >> 5)) * 512 + (size_t)((t & 15) + 16 * ((c >> 3) & 3)) * 8 + (c & 7);
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

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

template <typename T>
__device__ __forceinline__ T ldg_nt(const T *p) {
    return __builtin_nontemporal_load(p);
}

// A 16-byte weight-tile load (non-temporal) at byte offset off of the weight
// matrix, through a buffer resource: one 32-bit lane offset against a scalar
// base, where a pointer per lane costs 64-bit address arithmetic per load
// (one-token O 8.4 -> 7.9 us, QKV 12.6 -> 12.4 us).  Matrices stay below
// 2 GiB (checked at model load), so off fits the 32-bit offset.
__device__ __forceinline__ u32x4_t ldw(const void *w, size_t off) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(w), 0, 0x7fffffff, 0x00020000);
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2);
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
template <> struct WT_<W_Q8> { static constexpr int KSTEP = 64, U = 2; };

__device__ __forceinline__ bf16x8_t i8x8_to_bf16(uint32_t w0, uint32_t w1) {
    // |code| <= 127 has at most 7 significant bits: exact in bf16 (byte ->
    // f32 conversions, then packed f32 -> bf16 conversions)
    f32x8_t f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[i] = (float)(int8_t)(w0 >> (8 * i));
        f[4 + i] = (float)(int8_t)(w1 >> (8 * i));
    }
    return __builtin_convertvector(f, bf16x8_t);
}

// Weight codes as relaid at load (q + 128, sign bit flipped) -> bf16 q.
__device__ __forceinline__ bf16x8_t q8w_to_bf16(uint32_t w0, uint32_t w1) {
    return i8x8_to_bf16(w0 ^ 0x80808080u, w1 ^ 0x80808080u);
}

// Offset code u in [1, 255] -> the f16 value 1024 + u: u is the low mantissa
// byte under the exponent byte 0x64 (2^10, one unit per mantissa step), so
// one byte permute makes two values.  v_perm_b32 picks bytes 0-3 from its
// second operand and 4-7 from its first.
__device__ __forceinline__ f16x8_t u8x8_to_f16_1024(uint32_t w0, uint32_t w1) {
    u32x4_t r;
    r[0] = __builtin_amdgcn_perm(0x64646464u, w0, 0x04010400u);
    r[1] = __builtin_amdgcn_perm(0x64646464u, w0, 0x04030402u);
    r[2] = __builtin_amdgcn_perm(0x64646464u, w1, 0x04010400u);
    r[3] = __builtin_amdgcn_perm(0x64646464u, w1, 0x04030402u);
    return __builtin_bit_cast(f16x8_t, r);
}

// Element offset of the q8_0 scales of row block rb, k-step s (blocks 2s,
// 2s+1), lane group g: 8 f16 values, rows 4g..4g+3 of block 2s then of 2s+1.
__device__ __forceinline__ size_t q8_scale_ofs(int K, int rb, int s, int g) {
    return (((size_t)rb * (K / 64) + s) * 4 + g) * 8;
}

template <int WT, int RB>
struct StepIn {
    u32x4_t w[RB];
    u32x4_t xh, xl, xh2, xl2;          // bf16: xh/xl; q8: block 0 (xh, xl), block 1 (xh2, xl2); f32: xh
    u32x2_t sc[RB][2];                  // q8 scales of rows 4g..4g+3, blocks 2s, 2s+1
};

// One k-step's operands: the weight tile(s) from HBM and the activations of
// this lane's token, from global memory or (LDSB) from the normalised copy
// the fused-RMSNorm prologue left in LDS ([T][K] f32, or hi then lo planes).
template <int WT, int RB, bool LDSB>
__device__ __forceinline__ void load_step(const LinearArgs &a, const unsigned char *lds, int rb0, int s, int steps,
                                          int lane, int tok, bool tok_ok, StepIn<WT, RB> &in) {
    const int g = lane >> 4;
#pragma unroll
    for (int j = 0; j < RB; ++j) {
        const size_t tile = (size_t)s * (a.N / 16) + rb0 + j;      // k-step-major tiles
        in.w[j] = ldw(a.w, tile * 1024 + lane * 16);
    }
    const u32x4_t z = {0u, 0u, 0u, 0u};
    const size_t plane = (size_t)a.T * a.K;
    if (WT == W_F32) {
        const size_t o = (size_t)tok * (LDSB ? a.K : a.x.ld) + 16 * s + 4 * g;
        if (LDSB)
            in.xh = tok_ok ? *(const u32x4_t *)(lds + o * 4) : z;
        else
            in.xh = tok_ok ? *(const u32x4_t *)(a.x.f32 + o) : z;
    } else {
        const int kofs = (WT == W_BF16 ? 32 : 64) * s + 8 * g;
        const size_t o = (size_t)tok * (LDSB ? a.K : a.x.ld) + kofs;
        const uint16_t *hi = LDSB ? (const uint16_t *)lds : a.x.hi;
        const uint16_t *lo = LDSB ? (const uint16_t *)lds + plane : a.x.lo;
        in.xh = tok_ok ? *(const u32x4_t *)(hi + o) : z;
        in.xl = tok_ok ? *(const u32x4_t *)(lo + o) : z;
        if (WT == W_Q8) {
            in.xh2 = tok_ok ? *(const u32x4_t *)(hi + o + 32) : z;
            in.xl2 = tok_ok ? *(const u32x4_t *)(lo + o + 32) : z;
#pragma unroll
            for (int j = 0; j < RB; ++j) {
                const u32x4_t sv = *(const u32x4_t *)(a.wscale + q8_scale_ofs(a.K, rb0 + j, s, g));
                in.sc[j][0] = u32x2_t{sv[0], sv[1]};
                in.sc[j][1] = u32x2_t{sv[2], sv[3]};
            }
        }
    }
}

// load_step for a product that normalises its input on the fly (XN): the
// activations are the raw f32 rows of the residual times the norm gain,
// split into bf16 hi + lo planes in registers (f32 weights: used as they
// are); the token's 1/rms, whose sum of squares ss accumulates here over
// this lane's values, scales the sums in the epilogue.  The rows are
// a.norm.x (row map a.norm.rows).
template <int WT, int RB>
__device__ __forceinline__ void load_step_xn(const LinearArgs &a, int rb0, int s, int lane, int tok, bool tok_ok,
                                             StepIn<WT, RB> &in, float &ss) {
    const int g = lane >> 4;
#pragma unroll
    for (int j = 0; j < RB; ++j) {
        const size_t tile = (size_t)s * (a.N / 16) + rb0 + j;
        in.w[j] = ldw(a.w, tile * 1024 + lane * 16);
    }
    const float *xr = a.norm.x + (size_t)(a.norm.rows ? a.norm.rows[tok] : tok) * a.norm.ld;
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    // 8 values from k: x * gain as bf16 hi and lo planes
    auto split8 = [&](int k, u32x4_t &h, u32x4_t &l) {
        const f32x4_t x0 = tok_ok ? *(const f32x4_t *)(xr + k) : z, x1 = tok_ok ? *(const f32x4_t *)(xr + k + 4) : z;
        const f32x4_t g0 = *(const f32x4_t *)(a.norm.gain + k), g1 = *(const f32x4_t *)(a.norm.gain + k + 4);
        ss += x0[0] * x0[0] + x0[1] * x0[1] + x0[2] * x0[2] + x0[3] * x0[3] + x1[0] * x1[0] + x1[1] * x1[1] +
              x1[2] * x1[2] + x1[3] * x1[3];
        const f32x4_t y0 = x0 * g0, y1 = x1 * g1;
        uint16_t hh[8], ll[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float y = e < 4 ? y0[e] : y1[e - 4];
            hh[e] = f2bf(y);
            ll[e] = f2bf(y - bf2f(hh[e]));
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            h[e] = (uint32_t)hh[2 * e] | ((uint32_t)hh[2 * e + 1] << 16);
            l[e] = (uint32_t)ll[2 * e] | ((uint32_t)ll[2 * e + 1] << 16);
        }
    };
    if (WT == W_F32) {
        const int k = 16 * s + 4 * g;
        const f32x4_t x = tok_ok ? *(const f32x4_t *)(xr + k) : z;
        ss += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
        in.xh = __builtin_bit_cast(u32x4_t, x * *(const f32x4_t *)(a.norm.gain + k));
    } else {
        const int k = (WT == W_BF16 ? 32 : 64) * s + 8 * g;
        split8(k, in.xh, in.xl);
        if (WT == W_Q8) {
            split8(k + 32, in.xh2, in.xl2);
#pragma unroll
            for (int j = 0; j < RB; ++j) {
                const u32x4_t sv = *(const u32x4_t *)(a.wscale + q8_scale_ofs(a.K, rb0 + j, s, g));
                in.sc[j][0] = u32x2_t{sv[0], sv[1]};
                in.sc[j][1] = u32x2_t{sv[2], sv[3]};
            }
        }
    }
}

// OFS (q8_0, LDS-staged decode products): the codes (stored as q + 128)
// enter f16 MFMAs against f16 activation planes.
template <int WT, int RB, bool OFS = false>
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
    } else if (OFS) {
        // f16 activation planes; each code q becomes the f16 1024 + (q + 128)
        // by byte permutes, and q again (exact) by one packed f16 subtract
        const f16x8_t xh0 = __builtin_bit_cast(f16x8_t, in.xh);
        const f16x8_t xl0 = __builtin_bit_cast(f16x8_t, in.xl);
        const f16x8_t xh1 = __builtin_bit_cast(f16x8_t, in.xh2);
        const f16x8_t xl1 = __builtin_bit_cast(f16x8_t, in.xl2);
        const f16x8_t ofs = (_Float16)1152.0f;
        const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            const u32x4_t w = in.w[j];         // codes stored as q + 128
            const f16x8_t A0 = u8x8_to_f16_1024(w[0], w[1]) - ofs;
            const f16x8_t A1 = u8x8_to_f16_1024(w[2], w[3]) - ofs;
            f32x4_t d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, xh0, z, 0, 0, 0);
            d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, xl0, d0, 0, 0, 0);
            f32x4_t d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, xh1, z, 0, 0, 0);
            d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, xl1, d1, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t s0w = in.sc[j][0][i >> 1], s1w = in.sc[j][1][i >> 1];
                const float s0 = h2f((uint16_t)(s0w >> (16 * (i & 1))));
                const float s1 = h2f((uint16_t)(s1w >> (16 * (i & 1))));
                acc[j][i] = fmaf(s1, d1[i], fmaf(s0, d0[i], acc[j][i]));
            }
        }
    } else {
        const bf16x8_t xh0 = __builtin_bit_cast(bf16x8_t, in.xh);
        const bf16x8_t xl0 = __builtin_bit_cast(bf16x8_t, in.xl);
        const bf16x8_t xh1 = __builtin_bit_cast(bf16x8_t, in.xh2);
        const bf16x8_t xl1 = __builtin_bit_cast(bf16x8_t, in.xl2);
        const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            const bf16x8_t A0 = q8w_to_bf16(in.w[j][0], in.w[j][1]);
            const bf16x8_t A1 = q8w_to_bf16(in.w[j][2], in.w[j][3]);
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
// V cache element (cell c, dim d) inside one (stream, KV head) block of
// n_cells * hd elements: 32-cell tiles [c / 32][hd][32 slots], so a 32-cell
// step of attention reads one contiguous hd * 32 run.  Inside a tile, cell
// j sits in slot 8 * ((j & 15) >> 2) + 4 * (j >> 4) + (j & 3): the eight
// cells {4g..4g+3, 16+4g..16+4g+3} that one lane of the P*V product needs
// (see attn_mfma_kernel) are one 16-byte run.
__device__ __forceinline__ size_t v_off(int hd, int d, size_t c) {
    const int j = (int)(c & 31);
    return ((c >> 5) * hd + d) * 32 + 8 * ((j & 15) >> 2) + 4 * (j >> 4) + (j & 3);
}

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
        // n..n+3 stay contiguous in the tiled layout too (n is a multiple of 4)
        const size_t o = act_idx(a.out, t, n);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float gt = v[i], up = u[i];
            store_act(a.out, o + i, gt / (1.0f + expf(-gt)) * up);
        }
    } else if (EPI == EPI_QKV) {
        const QKVEpi &q = a.qkv;
        const int hd = q.head_dim;
        if (n < q.n_q_rows + q.n_k_rows) {
            const int base = n < q.n_q_rows ? 0 : q.n_q_rows;
            const int d = (n - base) % hd;       // a multiple of 4: two whole pairs, 16-byte aligned
            const float4 cs = *(const float4 *)(q.rope_cs + (size_t)t * (hd >> 1) + (d >> 1));
            const float c[2] = {cs.x, cs.z}, sf[2] = {cs.y, cs.w};
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
                const float x0 = v[2 * pr], x1 = v[2 * pr + 1];
                v[2 * pr] = x0 * c[pr] - x1 * sf[pr];
                v[2 * pr + 1] = x0 * sf[pr] + x1 * c[pr];
            }
        }
        if (n < q.n_q_rows) {
            store4(q.q_out + (size_t)t * q.n_q_rows + n, v);
        } else if (n < q.n_q_rows + q.n_k_rows && q.type_k == KV_Q8) {
            store4(q.kv_stage + (size_t)t * 2 * q.n_k_rows + (n - q.n_q_rows), v);
        } else if (n >= q.n_q_rows + q.n_k_rows && q.type_v == KV_Q8) {
            store4(q.kv_stage + (size_t)t * 2 * q.n_k_rows + (n - q.n_q_rows), v);
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
            const size_t base = ((size_t)a.tok.stream[t] * q.n_head_kv + head) * q.n_cells * hd;
            const int cell = a.tok.cell[t];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const size_t idx = base + v_off(hd, d + i, cell);
                if (q.type_v == KV_F32)
                    ((float *)q.v_cache)[idx] = v[i];
                else
                    ((uint16_t *)q.v_cache)[idx] = f2h(v[i]);
            }
        }
    }
}

// Fused RMSNorm of the (at most NORM_TMAX) input rows: every work-group
// reduces the rows' squares itself, then leaves x * rsqrt(mean(x^2) + eps)
// * gain in LDS in the format the MFMA B operand wants.
template <int WT, int NW>
__device__ void norm_prologue(const LinearArgs &a, unsigned char *lds) {
    // one pass: each thread keeps its slice of x in registers (K <= 8192
    // with 256+ threads -> at most 8 float4), reduces, then normalises it
    constexpr int TH = 64 * NW, MAXV = (8192 / 4 + TH - 1) / TH;
    __shared__ float red_ss[NORM_TMAX][NW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = a.K, T = a.T;
    f32x4_t v[NORM_TMAX][MAXV];
    for (int t = 0; t < T; ++t) {
        const float *xr = a.norm.x + (size_t)(a.norm.rows ? a.norm.rows[t] : t) * a.norm.ld;
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < MAXV; ++i) {
            const int e = (tid + TH * i) * 4;
            v[t][i] = e < K ? *(const f32x4_t *)(xr + e) : f32x4_t{0.f, 0.f, 0.f, 0.f};
            ss += v[t][i][0] * v[t][i][0] + v[t][i][1] * v[t][i][1] + v[t][i][2] * v[t][i][2] +
                  v[t][i][3] * v[t][i][3];
        }
        ss = wave_sum(ss);
        if (lane == 0) red_ss[t][wave] = ss;
    }
    __syncthreads();
    const size_t plane = (size_t)T * K;
    for (int t = 0; t < T; ++t) {
        float tot = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) tot += red_ss[t][w];
        const float inv = 1.0f / sqrtf(tot / (float)K + a.norm.eps);
#pragma unroll
        for (int i = 0; i < MAXV; ++i) {
            const int e = (tid + TH * i) * 4;
            if (e >= K) continue;
            const f32x4_t y = v[t][i] * inv * *(const f32x4_t *)(a.norm.gain + e);
            const size_t o = (size_t)t * K + e;
            if (WT == W_F32) {
                *(f32x4_t *)(lds + o * 4) = y;
            } else {
                u16x4_t hh, ll;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    hh[k] = f2bf(y[k]);
                    ll[k] = f2bf(y[k] - bf2f(hh[k]));
                }
                *(u16x4_t *)((uint16_t *)lds + o) = hh;
                *(u16x4_t *)((uint16_t *)lds + plane + o) = ll;
            }
        }
    }
    __syncthreads();
}

// RB row blocks per work-group share each k-step's activation fragment
// (SWIGLU: RB/2 gate|up pairs); KSPLIT > 1 (residual products only) splits
// k over grid.z and adds the partial sums atomically.  The input's RMSNorm
// fused: NORM stages the normalised rows in LDS (at most NORM_TMAX rows);
// XN normalises on the fly (load_step_xn), each work-group covering the
// whole k range of its rows and so the whole sum of squares of each token.
template <int WT, int EPI, int NW, bool NORM, int RB, int KSPLIT, bool XN = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(4))) void linear_small_kernel(LinearArgs a) {
    static_assert(EPI != EPI_SWIGLU || RB % 2 == 0, "gate|up pairs");
    static_assert(KSPLIT == 1 || EPI == EPI_RESID, "k split only for residual products");
    static_assert(!XN || (!NORM && KSPLIT == 1), "on-the-fly norm: whole k range per work-group");
    // k-steps per batch: the same 16-byte weight loads in flight per lane
    // (half with XN, whose f32 rows and gains take twice the registers)
    constexpr int U0 = WT_<WT>::U / RB > 0 ? WT_<WT>::U / RB : 1;
    constexpr int KSTEP = WT_<WT>::KSTEP, U = XN && U0 > 1 ? U0 / 2 : U0;
    extern __shared__ __align__(16) unsigned char dyn_lds[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int rb0 = blockIdx.x * RB;
    const int t0 = blockIdx.y * 16;
    const int n_tok = min(16, a.T - t0);
    const bool tok_ok = r < n_tok;
    const int tok = t0 + (tok_ok ? r : 0);
    const int steps = a.K / KSTEP;
    const int kz0 = blockIdx.z * steps / KSPLIT, kz1 = (blockIdx.z + 1) * steps / KSPLIT;
    const int s0 = kz0 + wave * (kz1 - kz0) / NW, s1 = kz0 + (wave + 1) * (kz1 - kz0) / NW;

    f32x4_t acc[RB];
#pragma unroll
    for (int j = 0; j < RB; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // with the fused norm, the first U weight tiles are requested before the
    // prologue so that HBM traffic overlaps the reduction
    constexpr int HOIST = U;
    u32x4_t w0[NORM ? HOIST : 1][RB];
    if (NORM) {
#pragma unroll
        for (int u = 0; u < HOIST; ++u)
#pragma unroll
            for (int j = 0; j < RB; ++j)
                if (s0 + u < s1)
                    w0[u][j] = ldw(a.w, ((size_t)(s0 + u) * (a.N / 16) + rb0 + j) * 1024 + lane * 16);
        norm_prologue<WT, NW>(a, dyn_lds);
    }

    float ss = 0.f;                                 // XN: this lane's share of its token's sum of squares
    for (int s = s0; s < s1; s += U) {
        StepIn<WT, RB> in[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (s + u < s1) {
                if constexpr (XN)
                    load_step_xn<WT, RB>(a, rb0, s + u, lane, tok, tok_ok, in[u], ss);
                else
                    load_step<WT, RB, NORM>(a, dyn_lds, rb0, s + u, steps, lane, tok, tok_ok, in[u]);
            }
        if (NORM && s == s0) {
#pragma unroll
            for (int u = 0; u < HOIST; ++u)
#pragma unroll
                for (int j = 0; j < RB; ++j) in[u].w[j] = w0[u][j];
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (s + u < s1) mfma_step<WT, RB>(in[u], acc);
    }

    __shared__ float red_ss[XN ? NW : 1][16];
    if (XN) {
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        if (lane < 16) red_ss[wave][lane] = ss;
    }
    if (NW > 1) {
        __shared__ f32x4_t red[NW > 1 ? NW - 1 : 1][RB][64];
        if (wave > 0) {
#pragma unroll
            for (int j = 0; j < RB; ++j) red[wave - 1][j][lane] = acc[j];
        }
        __syncthreads();
        if (wave != 0) return;
        // one wave's partial sums at a time (all of them at once would need
        // (NW - 1) * RB * 4 registers)
#pragma unroll 1
        for (int w = 0; w < NW - 1; ++w)
#pragma unroll
            for (int j = 0; j < RB; ++j) acc[j] += red[w][j][lane];
    } else if (XN) {
        __syncthreads();
    }
    if (!tok_ok) return;
    if (XN) {
        float tot = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) tot += red_ss[w][r];
        const float inv = 1.0f / sqrtf(tot / (float)a.K + a.norm.eps);
#pragma unroll
        for (int j = 0; j < RB; ++j) acc[j] *= inv;
    }
    const int t = t0 + r;
#pragma unroll
    for (int j = 0; j < RB; ++j) {
        if (EPI == EPI_SWIGLU) {
            if (j & 1) continue;
            epilogue4<EPI, false>(a, t, (rb0 / 2 + j / 2) * 16 + 4 * g, acc[j], acc[j + 1]);
        } else {
            epilogue4<EPI, (KSPLIT > 1)>(a, t, (rb0 + j) * 16 + 4 * g, acc[j], acc[j]);
        }
    }
}

// Few-token product with the activations in LDS (decode).  The work-group
// first requests its first batch of weight tiles, then copies (NORM:
// RMS-normalises) its <= 16 activation rows into LDS in the B-operand
// format, then streams weight tiles through two register buffers so the
// next batch is in flight while the current one is multiplied; B fragments
// are read from LDS right before use.  k-steps are split over NW waves and
// reduced through LDS (aliasing the activation copy).
// q8_0 scales: the batch needs UB * RB groups of 16 words (32 f16 scales of
// one row block and k-step: lane group g's 4 words are rows 4g..4g+3 of the
// step's two 32-wide blocks).  They are held one word per lane, each 16-lane
// row g holding its own group's words: lane 16g + 4c + i holds word i of
// group g for the batch's pair c = j UB + u (row block j, step u), so a step
// takes its 4 words by DPP row broadcasts, in the vector ALU (cross-lane
// permutes through LDS took the same 4 instructions per step, each an LDS
// round trip).  Kept whole in every lane, the scales took as many registers
// as the codes.
template <int WT, int RB, int UB>
struct WBatch {
    static_assert(WT != W_Q8 || UB * RB <= 4, "q8_0: one scale word per lane");
    u32x4_t w[UB][RB];
    uint32_t sc;
};

// this lane's scale word of the batch at k-step s (words past the wave's
// last step s1 are not loaded: no step reads them)
template <int RB, int UB>
__device__ __forceinline__ void load_wbatch_scales(const LinearArgs &a, int rb0, int s, int s1, int lane,
                                                   uint32_t &sc) {
    const int g = lane >> 4, c = (lane >> 2) & 3, i = lane & 3;
    const int j = c / UB, u = c % UB;
    const bool live = c < UB * RB && s + u < s1;
    const uint16_t *src = a.wscale + q8_scale_ofs(a.K, rb0 + (live ? j : 0), s + (live ? u : 0), g) + 2 * i;
    sc = live ? *(const uint32_t *)src : 0u;
}

// v of lane n (0..15) of this lane's 16-lane row (DPP row_newbcast; n a
// constant once the callers' loops are unrolled)
__device__ __forceinline__ uint32_t row_lane(uint32_t v, int n) {
    switch (n) {
#define UBD_ROW_LANE(N) \
    case N: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x150 + N, 0xF, 0xF, false);
        UBD_ROW_LANE(0) UBD_ROW_LANE(1) UBD_ROW_LANE(2) UBD_ROW_LANE(3)
        UBD_ROW_LANE(4) UBD_ROW_LANE(5) UBD_ROW_LANE(6) UBD_ROW_LANE(7)
        UBD_ROW_LANE(8) UBD_ROW_LANE(9) UBD_ROW_LANE(10) UBD_ROW_LANE(11)
        UBD_ROW_LANE(12) UBD_ROW_LANE(13) UBD_ROW_LANE(14) UBD_ROW_LANE(15)
#undef UBD_ROW_LANE
    }
    return 0u;
}

// row block j, step u of the batch: this lane's scales (rows 4g..4g+3 of
// blocks 2s and 2s + 1) are the words of lanes 4 (j UB + u) + q, q = 0..3,
// of its row
template <int RB, int UB>
__device__ __forceinline__ void wbatch_scales(uint32_t sc, int j, int u, u32x2_t &b0, u32x2_t &b1) {
    const int c = j * UB + u;
    b0 = u32x2_t{row_lane(sc, 4 * c), row_lane(sc, 4 * c + 1)};
    b1 = u32x2_t{row_lane(sc, 4 * c + 2), row_lane(sc, 4 * c + 3)};
}

template <int WT, int RB, int UB>
__device__ __forceinline__ void load_wbatch(const LinearArgs &a, int rb0, int s, int s1, int steps, int lane,
                                            WBatch<WT, RB, UB> &b) {
#pragma unroll
    for (int u = 0; u < UB; ++u) {
        if (s + u >= s1) break;
#pragma unroll
        for (int j = 0; j < RB; ++j)
            b.w[u][j] = ldw(a.w, ((size_t)(s + u) * (a.N / 16) + rb0 + j) * 1024 + lane * 16);
    }
    if constexpr (WT == W_Q8) load_wbatch_scales<RB, UB>(a, rb0, s, s1, lane, b.sc);
}

// load_wbatch for a batch known to be whole: no per-step exits, so the
// compiler sees a fixed count of loads after anything issued before them
template <int WT, int RB, int UB>
__device__ __forceinline__ void load_wbatch_whole(const LinearArgs &a, int rb0, int s, int lane,
                                                  WBatch<WT, RB, UB> &b) {
#pragma unroll
    for (int u = 0; u < UB; ++u)
#pragma unroll
        for (int j = 0; j < RB; ++j)
            b.w[u][j] = ldw(a.w, ((size_t)(s + u) * (a.N / 16) + rb0 + j) * 1024 + lane * 16);
    if constexpr (WT == W_Q8) load_wbatch_scales<RB, UB>(a, rb0, s, s + UB, lane, b.sc);
}

template <int WT, int RB, int UB>
__device__ __forceinline__ void mul_wbatch(const WBatch<WT, RB, UB> &b, const unsigned char *lds, int Tb, int K,
                                           int s, int s1, int lane, int tok, bool tok_ok, f32x4_t *acc) {
    const int g = lane >> 4;
    const size_t plane = (size_t)Tb * K;
#pragma unroll
    for (int u = 0; u < UB; ++u) {
        if (s + u >= s1) break;
        StepIn<WT, RB> in;
#pragma unroll
        for (int j = 0; j < RB; ++j) in.w[j] = b.w[u][j];
        // lanes past the block's tokens read token 0: their output columns
        // are never stored, so no masking
        (void)tok_ok;
        if (WT == W_F32) {
            in.xh = *(const u32x4_t *)(lds + ((size_t)tok * K + 16 * (s + u) + 4 * g) * 4);
        } else {
            const size_t o = (size_t)tok * K + (WT == W_BF16 ? 32 : 64) * (s + u) + 8 * g;
            const uint16_t *hi = (const uint16_t *)lds, *lo = (const uint16_t *)lds + plane;
            in.xh = *(const u32x4_t *)(hi + o);
            in.xl = *(const u32x4_t *)(lo + o);
            if constexpr (WT == W_Q8) {
                in.xh2 = *(const u32x4_t *)(hi + o + 32);
                in.xl2 = *(const u32x4_t *)(lo + o + 32);
#pragma unroll
                for (int j = 0; j < RB; ++j) wbatch_scales<RB, UB>(b.sc, j, u, in.sc[j][0], in.sc[j][1]);
            }
        }
        mfma_step<WT, RB, WT == W_Q8>(in, acc);
    }
}

// Activation copy of the LDS-staged product.  Every thread handles float4
// slices e = (tid + TH * i) * 4 of a row, CH slices at a time: the CH loads
// of a chunk are issued together and waited for once (a per-slice loop
// waited for every load, and so for the weight batches issued before it).
template <int WT, int NW, bool NORM>
__device__ int ldsx_prologue(const LinearArgs &a, unsigned char *lds, int t0, int Tb) {
    constexpr int TH = 64 * NW, CH = 4;
    int big = 0;
    __shared__ float red_ss[16][NW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = a.K;
    const size_t plane = (size_t)Tb * K;
    const int nv = (K / 4 + TH - 1) / TH;     // float4 slices per thread per row
    const f32x4_t z4 = {0.f, 0.f, 0.f, 0.f};
    float inv[16];
    if (NORM) {
        for (int t = 0; t < Tb; ++t) {
            const float *xr = a.norm.x + (size_t)(a.norm.rows ? a.norm.rows[t0 + t] : t0 + t) * a.norm.ld;
            float ss = 0.f;
            for (int i0 = 0; i0 < nv; i0 += CH) {
                f32x4_t v[CH];
#pragma unroll
                for (int i = 0; i < CH; ++i) {
                    const int e = (tid + TH * (i0 + i)) * 4;
                    v[i] = (i0 + i < nv && e < K) ? *(const f32x4_t *)(xr + e) : z4;
                }
#pragma unroll
                for (int i = 0; i < CH; ++i) ss += v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] + v[i][3] * v[i][3];
            }
            ss = wave_sum(ss);
            if (lane == 0) red_ss[t][wave] = ss;
        }
        __syncthreads();
        for (int t = 0; t < Tb; ++t) {
            float tot = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) tot += red_ss[t][w];
            inv[t] = 1.0f / sqrtf(tot / (float)K + a.norm.eps);
        }
    }
    for (int t = 0; t < Tb; ++t) {
        const float *xr = NORM ? a.norm.x + (size_t)(a.norm.rows ? a.norm.rows[t0 + t] : t0 + t) * a.norm.ld
                               : nullptr;
        for (int i0 = 0; i0 < nv; i0 += CH) {
            if (NORM) {
                f32x4_t v[CH], gn[CH];
#pragma unroll
                for (int i = 0; i < CH; ++i) {
                    const int e = (tid + TH * (i0 + i)) * 4;
                    const bool ok = i0 + i < nv && e < K;
                    v[i] = ok ? *(const f32x4_t *)(xr + e) : z4;
                    gn[i] = ok ? *(const f32x4_t *)(a.norm.gain + e) : z4;
                }
#pragma unroll
                for (int i = 0; i < CH; ++i) {
                    const int e = (tid + TH * (i0 + i)) * 4;
                    if (i0 + i >= nv || e >= K) continue;
                    const size_t o = (size_t)t * K + e;
                    const f32x4_t y = v[i] * inv[t] * gn[i];
                    if (WT == W_F32) {
                        *(f32x4_t *)(lds + o * 4) = y;
                    } else {
                        u16x4_t hh, ll;
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            uint16_t h1, l1;
                            split_hilo<WT>(y[k], h1, l1, big);
                            hh[k] = h1;
                            ll[k] = l1;
                        }
                        *(u16x4_t *)((uint16_t *)lds + o) = hh;
                        *(u16x4_t *)((uint16_t *)lds + plane + o) = ll;
                    }
                }
            } else if (WT == W_F32) {
                f32x4_t v[CH];
#pragma unroll
                for (int i = 0; i < CH; ++i) {
                    const int e = (tid + TH * (i0 + i)) * 4;
                    v[i] = (i0 + i < nv && e < K) ? *(const f32x4_t *)(a.x.f32 + (size_t)(t0 + t) * a.x.ld + e) : z4;
                }
#pragma unroll
                for (int i = 0; i < CH; ++i) {
                    const int e = (tid + TH * (i0 + i)) * 4;
                    if (i0 + i < nv && e < K) *(f32x4_t *)(lds + ((size_t)t * K + e) * 4) = v[i];
                }
            } else {
                u16x4_t h[CH], l[CH];
                const u16x4_t z = {0, 0, 0, 0};
#pragma unroll
                for (int i = 0; i < CH; ++i) {
                    const int e = (tid + TH * (i0 + i)) * 4;
                    const bool ok = i0 + i < nv && e < K;
                    const size_t src = (size_t)(t0 + t) * a.x.ld + e;
                    h[i] = ok ? *(const u16x4_t *)(a.x.hi + src) : z;
                    l[i] = ok ? *(const u16x4_t *)(a.x.lo + src) : z;
                }
#pragma unroll
                for (int i = 0; i < CH; ++i) {
                    const int e = (tid + TH * (i0 + i)) * 4;
                    if (i0 + i >= nv || e >= K) continue;
                    const size_t o = (size_t)t * K + e;
                    u16x4_t hh = h[i], ll = l[i];
                    if (WT == W_Q8) {
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            uint16_t h1, l1;
                            split_hilo<WT>(bf2f(h[i][k]) + bf2f(l[i][k]), h1, l1, big);
                            hh[k] = h1;
                            ll[k] = l1;
                        }
                    }
                    *(u16x4_t *)((uint16_t *)lds + o) = hh;
                    *(u16x4_t *)((uint16_t *)lds + plane + o) = ll;
                }
            }
        }
    }
    return copy_barrier<WT>(big);
}

// One-token variant of the activation copy, split in two so that the
// activation loads go out before the weight batches.  A wave's vector loads
// complete in issue order, so a copy issued after the weights (as above)
// cannot start before every weight of the wave's first two batches has
// arrived; issued first, it overlaps them.  Each thread keeps at most EVM
// float4 slices (and the gain's) in registers; longer rows use the copy
// above.
template <int WT, int NW> constexpr int evm() { return 4; }

template <int WT, bool NORM, int EVM>
struct EarlyX {
    f32x4_t v[WT == W_F32 || NORM ? EVM : 1];
    f32x4_t gn[NORM ? EVM : 1];
    u16x4_t h[WT == W_F32 || NORM ? 1 : EVM], l[WT == W_F32 || NORM ? 1 : EVM];
};

// one token, a row short enough for the registers, and a whole first
// weight batch for every wave
template <int WT, int NW, int UB>
__device__ __forceinline__ bool ldsx_early_fits(int K, int Tb, int steps) {
    return Tb == 1 && (K / 4 + 64 * NW - 1) / (64 * NW) <= evm<WT, NW>() && steps >= NW * UB;
}

template <int WT, int NW, bool NORM>
__device__ __forceinline__ void ldsx_early_load(const LinearArgs &a, int t0, EarlyX<WT, NORM, evm<WT, NW>()> &x) {
    constexpr int EVM = evm<WT, NW>();
    constexpr int TH = 64 * NW;
    const int tid = threadIdx.x, K = a.K;
    const f32x4_t z4 = {0.f, 0.f, 0.f, 0.f};
    const u16x4_t z = {0, 0, 0, 0};
    if (NORM) {
        const float *xr = a.norm.x + (size_t)(a.norm.rows ? a.norm.rows[t0] : t0) * a.norm.ld;
#pragma unroll
        for (int i = 0; i < EVM; ++i) {
            const int e = (tid + TH * i) * 4;
            x.v[i] = e < K ? *(const f32x4_t *)(xr + e) : z4;
            x.gn[i] = e < K ? *(const f32x4_t *)(a.norm.gain + e) : z4;
        }
    } else if (WT == W_F32) {
#pragma unroll
        for (int i = 0; i < EVM; ++i) {
            const int e = (tid + TH * i) * 4;
            x.v[i] = e < K ? *(const f32x4_t *)(a.x.f32 + (size_t)t0 * a.x.ld + e) : z4;
        }
    } else {
#pragma unroll
        for (int i = 0; i < EVM; ++i) {
            const int e = (tid + TH * i) * 4;
            const size_t src = (size_t)t0 * a.x.ld + e;
            x.h[i] = e < K ? *(const u16x4_t *)(a.x.hi + src) : z;
            x.l[i] = e < K ? *(const u16x4_t *)(a.x.lo + src) : z;
        }
    }
}

template <int WT, int NW, bool NORM>
__device__ int ldsx_early_store(const LinearArgs &a, unsigned char *lds, const EarlyX<WT, NORM, evm<WT, NW>()> &x) {
    constexpr int EVM = evm<WT, NW>();
    constexpr int TH = 64 * NW;
    int big = 0;
    __shared__ float red_ss[NW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = a.K;
    const size_t plane = (size_t)K;
    float inv = 1.f;
    if (NORM) {
        // the same summation order as the copy above (slices in order,
        // zeros past the row end)
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < EVM; ++i)
            ss += x.v[i][0] * x.v[i][0] + x.v[i][1] * x.v[i][1] + x.v[i][2] * x.v[i][2] + x.v[i][3] * x.v[i][3];
        ss = wave_sum(ss);
        if (lane == 0) red_ss[wave] = ss;
        __syncthreads();
        float tot = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) tot += red_ss[w];
        inv = 1.0f / sqrtf(tot / (float)K + a.norm.eps);
    }
#pragma unroll
    for (int i = 0; i < EVM; ++i) {
        const int e = (tid + TH * i) * 4;
        if (e >= K) continue;
        if (NORM || WT == W_F32) {
            const f32x4_t y = NORM ? x.v[i] * inv * x.gn[i] : x.v[i];
            if (WT == W_F32) {
                *(f32x4_t *)(lds + (size_t)e * 4) = y;
            } else {
                u16x4_t hh, ll;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    uint16_t h1, l1;
                    split_hilo<WT>(y[k], h1, l1, big);
                    hh[k] = h1;
                    ll[k] = l1;
                }
                *(u16x4_t *)((uint16_t *)lds + e) = hh;
                *(u16x4_t *)((uint16_t *)lds + plane + e) = ll;
            }
        } else {
            u16x4_t hh = x.h[i], ll = x.l[i];
            if (WT == W_Q8) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    uint16_t h1, l1;
                    split_hilo<WT>(bf2f(x.h[i][k]) + bf2f(x.l[i][k]), h1, l1, big);
                    hh[k] = h1;
                    ll[k] = l1;
                }
            }
            *(u16x4_t *)((uint16_t *)lds + e) = hh;
            *(u16x4_t *)((uint16_t *)lds + plane + e) = ll;
        }
    }
    return copy_barrier<WT>(big);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// q8_0 products whose activation copy met a value beyond the f16 planes
// (rare: only rows of very large activations).  Every row is formed again
// from its source, then stored scaled by 2^-e(t), with e(t) >= 0 the
// smallest exponent that brings the row's largest magnitude to at most
// 2^15; xs[t] = 2^e(t), by which the epilogue multiplies the token's sums.
// Scaling by a power of two is exact, so the products stay those of the
// unscaled values.
template <int NW, bool NORM>
__device__ __forceinline__ void ldsx_rescale(const LinearArgs &a, unsigned char *lds, int t0, int Tb, float *xs) {
    constexpr int TH = 64 * NW;
    __shared__ float red[NW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = a.K;
    const size_t plane = (size_t)Tb * K;
    for (int t = 0; t < Tb; ++t) {
        const float *xr = NORM ? a.norm.x + (size_t)(a.norm.rows ? a.norm.rows[t0 + t] : t0 + t) * a.norm.ld
                               : nullptr;
        float inv = 1.f;
        if (NORM) {
            float ss = 0.f;
            for (int e = tid * 4; e < K; e += TH * 4) {
                const f32x4_t v = *(const f32x4_t *)(xr + e);
                ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
            }
            ss = wave_sum(ss);
            if (lane == 0) red[wave] = ss;
            __syncthreads();
            float tot = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) tot += red[w];
            inv = 1.0f / sqrtf(tot / (float)K + a.norm.eps);
            __syncthreads();
        }
        auto row4 = [&](int e) -> f32x4_t {
            if (NORM) return *(const f32x4_t *)(xr + e) * inv * *(const f32x4_t *)(a.norm.gain + e);
            const size_t src = (size_t)(t0 + t) * a.x.ld + e;
            const u16x4_t h = *(const u16x4_t *)(a.x.hi + src), l = *(const u16x4_t *)(a.x.lo + src);
            return f32x4_t{bf2f(h[0]) + bf2f(l[0]), bf2f(h[1]) + bf2f(l[1]), bf2f(h[2]) + bf2f(l[2]),
                           bf2f(h[3]) + bf2f(l[3])};
        };
        float m = 0.f;
        for (int e = tid * 4; e < K; e += TH * 4) {
            const f32x4_t y = row4(e);
            m = fmaxf(m, fmaxf(fmaxf(fabsf(y[0]), fabsf(y[1])), fmaxf(fabsf(y[2]), fabsf(y[3]))));
        }
        m = wave_max(m);
        if (lane == 0) red[wave] = m;
        __syncthreads();
        float mx = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) mx = fmaxf(mx, red[w]);
        int ex = 0;
        if (mx < INFINITY) (void)frexpf(mx, &ex);   // mx = f * 2^ex, f in [0.5, 1)
        const int sh = max(0, ex - 15);
        const float down = ldexpf(1.f, -sh);
        if (tid == 0) xs[t] = ldexpf(1.f, sh);
        for (int e = tid * 4; e < K; e += TH * 4) {
            const f32x4_t y = row4(e) * down;
            u16x4_t hh, ll;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                hh[k] = f2h(y[k]);
                ll[k] = f2h(y[k] - h2f(hh[k]));
            }
            *(u16x4_t *)((uint16_t *)lds + (size_t)t * K + e) = hh;
            *(u16x4_t *)((uint16_t *)lds + plane + (size_t)t * K + e) = ll;
        }
        __syncthreads();
    }
}

// 4 waves per SIMD (at most 128 registers).
template <int WT, int EPI, int NW, bool NORM>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(4)))
void linear_ldsx_kernel(LinearArgs a) {
    constexpr int RB = EPI == EPI_SWIGLU ? 2 : 1;
    constexpr int KSTEP = WT_<WT>::KSTEP;
    // k-steps per weight batch: 8 tiles per batch; q8_0: 2 k-steps, 4 for the
    // logits (each wave's k range of the narrower q8_0 products is in flight
    // whole with two 2-step batches; longer batches made them slower: down
    // 17.3 -> 21.2 us, O 9.7 -> 11.0, QKV 12.3 -> 13.4 at config 5, logits
    // 100.4 -> 96.0)
    constexpr int UB = WT == W_Q8 ? (EPI == EPI_LOGITS ? 4 : 2) : 8 / RB;
    extern __shared__ __align__(16) unsigned char dyn_lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int rb0 = blockIdx.x * RB;
    const int t0 = blockIdx.y * 16;
    const int Tb = min(16, a.T - t0);
    const bool tok_ok = r < Tb;
    const int tok = tok_ok ? r : 0;                 // row within the LDS copy
    const int steps = a.K / KSTEP;
    const int s0 = wave * steps / NW, s1 = (wave + 1) * steps / NW;

    f32x4_t acc[RB];
#pragma unroll
    for (int j = 0; j < RB; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // both weight batches go out before the prologue, and each is refilled
    // right after it has been multiplied: two batches stay in flight
    WBatch<WT, RB, UB> bufA, bufB;
    int big;                                        // q8_0: a value beyond the f16 planes
    if (a.early && ldsx_early_fits<WT, NW, UB>(a.K, Tb, steps)) {
        EarlyX<WT, NORM, evm<WT, NW>()> x;
        ldsx_early_load<WT, NW, NORM>(a, t0, x);
        asm volatile("" ::: "memory");              // activation loads first
        load_wbatch_whole<WT, RB, UB>(a, rb0, s0, lane, bufA);
        if (s0 + UB < s1) load_wbatch<WT, RB, UB>(a, rb0, s0 + UB, s1, steps, lane, bufB);
        big = ldsx_early_store<WT, NW, NORM>(a, dyn_lds, x);
    } else {
        if (s0 < s1) load_wbatch<WT, RB, UB>(a, rb0, s0, s1, steps, lane, bufA);
        if (s0 + UB < s1) load_wbatch<WT, RB, UB>(a, rb0, s0 + UB, s1, steps, lane, bufB);
        big = ldsx_prologue<WT, NW, NORM>(a, dyn_lds, t0, Tb);
    }
    __shared__ float xs[WT == W_Q8 ? 16 : 1];      // per-token scale of a rescaled copy
    if (WT == W_Q8 && big) {
        ldsx_rescale<NW, NORM>(a, dyn_lds, t0, Tb, xs);
        // both batches are requested again: their first copies are then dead
        // during the rescale, which can use their registers
        if (s0 < s1) load_wbatch<WT, RB, UB>(a, rb0, s0, s1, steps, lane, bufA);
        if (s0 + UB < s1) load_wbatch<WT, RB, UB>(a, rb0, s0 + UB, s1, steps, lane, bufB);
    }
    for (int s = s0; s < s1; s += 2 * UB) {
        mul_wbatch<WT, RB, UB>(bufA, dyn_lds, Tb, a.K, s, s1, lane, tok, tok_ok, acc);
        if (s + 2 * UB < s1) load_wbatch<WT, RB, UB>(a, rb0, s + 2 * UB, s1, steps, lane, bufA);
        if (s + UB >= s1) break;
        mul_wbatch<WT, RB, UB>(bufB, dyn_lds, Tb, a.K, s + UB, s1, lane, tok, tok_ok, acc);
        if (s + 3 * UB < s1) load_wbatch<WT, RB, UB>(a, rb0, s + 3 * UB, s1, steps, lane, bufB);
    }

    if (NW > 1) {
        __syncthreads();                            // everyone is done with the activation copy
        f32x4_t *red = (f32x4_t *)dyn_lds;          // [NW-1][RB][64]
        if (wave > 0) {
#pragma unroll
            for (int j = 0; j < RB; ++j) red[((wave - 1) * RB + j) * 64 + lane] = acc[j];
        }
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int w = 0; w < NW - 1; ++w)
#pragma unroll
            for (int j = 0; j < RB; ++j) acc[j] += red[(w * RB + j) * 64 + lane];
    }
    if (!tok_ok) return;
    if (WT == W_Q8 && big) {
        const float f = xs[r];
#pragma unroll
        for (int j = 0; j < RB; ++j) acc[j] *= f;
    }
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
                        wr[i][j] = ldw(a.w, ((size_t)(2 * st + j) * nrb + rb) * 1024 + lane * 16);
                } else {
                    wr[i][0] = ldw(a.w, ((size_t)st * nrb + rb) * 1024 + lane * 16);
                    const u32x4_t sv = *(const u32x4_t *)(a.wscale + q8_scale_ofs(a.K, rb, st, g));
                    sc[i][0] = u32x2_t{sv[0], sv[1]};
                    sc[i][1] = u32x2_t{sv[2], sv[3]};
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
                A[i][0] = q8w_to_bf16(wr[i][0][0], wr[i][0][1]);
                A[i][1] = q8w_to_bf16(wr[i][0][2], wr[i][0][3]);
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

// ---------------------------------------------------------------------------
// Prefill product with an LDS ring of activation stages.  A work-group of 4
// waves owns 64*RBW weight rows x 16*TB tokens; wave w owns row blocks
// rb0 + w*RBW ...  The k range is walked in stages of KS values.  Weight
// tiles (already in MFMA fragment order) stream into registers one stage
// ahead; activation fragments are copied by every wave, a quarter each,
// straight from global memory into a 3-deep LDS ring (buffer_load ... lds,
// 16 bytes per lane, fragment order) two stages ahead.  One barrier per
// stage, after each wave has waited for its own copies of that stage.

// Raw buffer resource over `bytes` bytes at p (gfx9 descriptor: 32-bit
// data format word; loads beyond num_records return zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, size_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)min(bytes, (size_t)0x7fffffff), 0x00020000);
}

// s_waitcnt immediate (gfx9 encoding) that bounds only the vector-memory
// counter: at most N vector loads of this wave still outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Work-group barrier that leaves the memory counters to the caller; the
// empty asm statements stop the compiler from moving memory accesses across.
__device__ __forceinline__ void wg_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int WT, int RBW, int TB, int KS, bool LO = false> struct GemmCfg {
    static constexpr bool Q8 = WT == W_Q8;
    static constexpr int PL = Q8 || LO ? 2 : 1;   // activation planes: hi (+ lo for q8_0, or bf16 with LO)
    static constexpr int KH = KS / 32;            // 32-wide k halves per stage
    static constexpr int NA = Q8 ? KS / 64 : KH;  // weight tiles per row block per stage
    static constexpr int XF = TB * KH * PL;       // activation fragments per stage
    static_assert(KS % 64 == 0 && XF % 4 == 0, "stage shape");
    static constexpr int XW = XF / 4;             // ... copied by each wave
    static constexpr int NX = 3;                  // LDS ring depth
};

// LO (bf16 weights): the activations' lo plane enters a second product per
// fragment, so the product sees about 16 significant bits of the f32
// activation instead of bf16's 8.
template <int WT, int EPI, int RBW, int TB, int SPLITK, int KS, int WPD, bool LO = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void gemm_lds_kernel(LinearArgs a,
                                                                                             int n_wtiles,
                                                                                             int n_ttiles) {
    // (the host pass only needs the launch stub; the buffer-resource
    // builtins below exist for the device pass alone)
#if defined(__HIP_DEVICE_COMPILE__)
    using C = GemmCfg<WT, RBW, TB, KS, LO>;
    constexpr bool Q8 = C::Q8;
    constexpr int KH = C::KH, NA = C::NA;
    __shared__ u32x4_t xs[C::NX * C::XF * 64];

    const int lane = threadIdx.x & 63;
    // wave-uniform (scalar) wave index: the LDS destination of the copies
    // goes through M0 and must be uniform
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int total = n_wtiles * n_ttiles * SPLITK;
    const int b = blockIdx.x;
    // consecutive tiles (same weight rows, next token block) on one XCD
    const int tile = (total % 8 == 0) ? (b % 8) * (total / 8) + b / 8 : b;
    const int ks = tile % SPLITK;
    const int tt = (tile / SPLITK) % n_ttiles;
    const int nt = tile / (SPLITK * n_ttiles);
    const int nrb = a.N / 16;
    const int rb0 = nt * 4 * RBW + wave * RBW;
    const int t0 = tt * 16 * TB;
    const int nstage = a.K / KS;
    const int st0 = ks * nstage / SPLITK, st1 = (ks + 1) * nstage / SPLITK;
    const int KB = a.K / 32;

    // Buffer resources (bounds-checked: offsets past num_records read 0, so
    // token rows past T need no clamping).  Every load is a loop-invariant
    // 32-bit lane offset plus a per-stage scalar offset.
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, (size_t)a.N * a.K * (Q8 ? 1 : 2));
    // (tiled activations: whole 16-token tiles, each fragment one
    // contiguous 1 KB run; row-major: 16 rows x 64 bytes per fragment)
    const size_t xbytes = (size_t)(a.x.tiled ? (a.T + 15) / 16 * 16 : a.T) * a.x.ld * 2;
    const __amdgpu_buffer_rsrc_t rxh = make_rsrc(a.x.hi, xbytes);
    const __amdgpu_buffer_rsrc_t rxl = make_rsrc(C::PL == 2 ? a.x.lo : a.x.hi, xbytes);
    const __amdgpu_buffer_rsrc_t rsc = make_rsrc(a.wscale, Q8 ? (size_t)a.N * KB * 2 : 0);
    const int xst = a.x.tiled ? KS * 32 : KS * 2;     // bytes between stages
    // this wave's activation fragments f = wave*XW + u = (plane, token block, k half)
    int xoff[C::XW];
#pragma unroll
    for (int u = 0; u < C::XW; ++u) {
        const int f = wave * C::XW + u;
        const int tb = (f / KH) % TB, j = f % KH;
        xoff[u] = a.x.tiled ? ((t0 / 16 + tb) * (a.x.ld / 32) + j) * 1024 + lane * 16
                            : ((t0 + 16 * tb + r) * a.x.ld + 32 * j + 8 * g) * 2;
    }
    // weight row blocks past N re-read the last one (never stored)
    int woff[RBW], soff[RBW];
#pragma unroll
    for (int i = 0; i < RBW; ++i) {
        const int rbc = min(rb0 + i, nrb - 1);
        woff[i] = rbc * 1024 + lane * 16;
        soff[i] = (int)q8_scale_ofs(a.K, rbc, 0, g) * 2;
    }
    const int wstep = nrb * 1024;   // bytes between consecutive k-steps of the weight tiles

    // weight tiles of the next WPD stages (in flight): one register set per
    // stage of look-ahead, used in turn
    u32x4_t wn0[RBW][NA], wn1[RBW][NA];
    u32x2_t sn0[RBW][KH], sn1[RBW][KH];     // ... and q8_0 scales
    static_assert(!Q8 || KH % 2 == 0, "q8_0 scales load in pairs of 32-blocks");
    constexpr int NWL = RBW * NA + (Q8 ? RBW * KH / 2 : 0);   // weight loads per stage
    f32x4_t acc[RBW][TB];
#pragma unroll
    for (int i = 0; i < RBW; ++i)
#pragma unroll
        for (int j = 0; j < TB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto issue_w = [&](int s, u32x4_t (&wn)[RBW][NA], u32x2_t (&sn)[RBW][KH]) {
#pragma unroll
        for (int j = 0; j < NA; ++j) {
            const int so = (NA * s + j) * wstep;
#pragma unroll
            for (int i = 0; i < RBW; ++i) wn[i][j] = __builtin_amdgcn_raw_buffer_load_b128(rw, woff[i], so, 0);
        }
        if (Q8) {
#pragma unroll
            for (int i = 0; i < RBW; ++i)
#pragma unroll
                for (int j = 0; j < KH; j += 2) {
                    // blocks KH s + j and + 1: 64-wide k-step (KH s + j) / 2
                    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rsc, soff[i], (KH * s + j) / 2 * 64, 0);
                    sn[i][j] = u32x2_t{v[0], v[1]};
                    sn[i][j + 1] = u32x2_t{v[2], v[3]};
                }
        }
    };
    // stage s's activation copies into ring slot s % NX (stage clamped)
    auto issue_x = [&](int s) {
        const int sl = min(s, st1 - 1);
        u32x4_t *dst = xs + (size_t)((s % C::NX) * C::XF + wave * C::XW) * 64;
#pragma unroll
        for (int u = 0; u < C::XW; ++u) {
            const bool lo = (wave * C::XW + u) >= TB * KH;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(lo ? rxl : rxh,
                                                     (__attribute__((address_space(3))) void *)(dst + u * 64), 16,
                                                     xoff[u], sl * xst, 0, 0);
        }
    };

    auto stage = [&](int s, u32x4_t (&wn)[RBW][NA], u32x2_t (&sn)[RBW][KH]) {
            // landed: everything but the loads issued for the following
            // stage (its activation copies, and with WPD 2 its weights)
            wait_vm<WPD == 1 ? C::XW : C::XW + NWL>();
            wg_barrier();
            u32x4_t wc[RBW][NA];
            u32x2_t sc[RBW][KH];
#pragma unroll
            for (int i = 0; i < RBW; ++i) {
#pragma unroll
                for (int j = 0; j < NA; ++j) wc[i][j] = wn[i][j];
#pragma unroll
                for (int j = 0; j < KH; ++j) sc[i][j] = sn[i][j];
            }
            __builtin_amdgcn_sched_barrier(0);
            issue_w(min(s + WPD, st1 - 1), wn, sn);
            issue_x(s + 2);
            const u32x4_t *xb = xs + (size_t)(s % C::NX) * C::XF * 64;
#pragma unroll
            for (int j = 0; j < KH; ++j) {
                bf16x8_t Bh[TB];
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) Bh[tb] = __builtin_bit_cast(bf16x8_t, xb[(tb * KH + j) * 64 + lane]);
                if (!Q8) {
                    bf16x8_t Bl[LO ? TB : 1];
                    if (LO) {
#pragma unroll
                        for (int tb = 0; tb < TB; ++tb)
                            Bl[tb] = __builtin_bit_cast(bf16x8_t, xb[((TB + tb) * KH + j) * 64 + lane]);
                    }
#pragma unroll
                    for (int i = 0; i < RBW; ++i) {
                        const bf16x8_t A = __builtin_bit_cast(bf16x8_t, wc[i][j]);
#pragma unroll
                        for (int tb = 0; tb < TB; ++tb) {
                            acc[i][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bh[tb], acc[i][tb], 0, 0, 0);
                            if (LO)
                                acc[i][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bl[tb], acc[i][tb], 0, 0, 0);
                        }
                    }
                } else {
                    const f32x4_t zf = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int i = 0; i < RBW; ++i) {
                        const u32x4_t w = wc[i][j >> 1];
                        const bf16x8_t A = (j & 1) ? q8w_to_bf16(w[2], w[3]) : q8w_to_bf16(w[0], w[1]);
                        f32x4_t S;
#pragma unroll
                        for (int e = 0; e < 4; ++e) S[e] = h2f((uint16_t)(sc[i][j][e >> 1] >> (16 * (e & 1))));
#pragma unroll
                        for (int tb = 0; tb < TB; ++tb) {
                            const bf16x8_t Bl =
                                __builtin_bit_cast(bf16x8_t, xb[((TB + tb) * KH + j) * 64 + lane]);
                            f32x4_t d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bh[tb], zf, 0, 0, 0);
                            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bl, d, 0, 0, 0);
                            acc[i][tb] += S * d;
                        }
                    }
                }
            }
            {
                // the stage's loads spread over its first products (2 loads, then
                // 4 products): issued as one burst by every wave after the
                // barrier, they filled the address queue and held the matrix
                // cores idle
                __builtin_amdgcn_sched_group_barrier(0x100, TB, 0);
#pragma unroll
                for (int q = 0; q < (NWL + C::XW + 3) / 4; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x010, 4, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                }
            }
    };
    if (st0 < st1) {
        issue_w(st0, wn0, sn0);
        issue_x(st0);
        if (WPD == 2) issue_w(min(st0 + 1, st1 - 1), wn1, sn1);
        issue_x(st0 + 1);
        if (WPD == 2) {
            for (int s = st0; s < st1; s += 2) {
                stage(s, wn0, sn0);
                if (s + 1 < st1) stage(s + 1, wn1, sn1);
            }
        } else {
            for (int s = st0; s < st1; ++s) stage(s, wn0, sn0);
        }
        // the ring's last copies must land before the work-group's LDS is released
        wait_vm<0>();
    }

#pragma unroll
    for (int i = 0; i < RBW; ++i) {
        const int rb = rb0 + i;
        if (rb >= nrb) continue;
        if (EPI == EPI_SWIGLU && (i & 1)) continue;
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const int t = t0 + tb * 16 + r;
            if (t >= a.T) continue;
            if (SPLITK > 1)
                store4(a.split_out + ((size_t)ks * a.T + t) * a.N + rb * 16 + 4 * g, acc[i][tb]);
            else if (EPI == EPI_SWIGLU)
                epilogue4<EPI, false>(a, t, (rb >> 1) * 16 + 4 * g, acc[i][tb], acc[i + 1][tb]);
            else
                epilogue4<EPI, false>(a, t, rb * 16 + 4 * g, acc[i][tb], acc[i][tb]);
        }
    }
#endif
}

// Deep variant of the LDS-ring product: weights D stages ahead in D + 1
// rotating register sets, activations XA stages ahead in an (XA + 1)-deep
// LDS ring.  The stage loop is unrolled by D + 1 and has no branches inside,
// so every register set is loaded and consumed at fixed places and no set
// is ever copied (a copy of a set still in flight makes the compiler wait
// for it, which leaves one stage's compute to cover a whole memory round
// trip).  OCC = waves per SIMD (1: the accumulators go to the matrix-core
// registers, leaving room for more sets).  bf16 weights; the stage count
// K / 64 must be a multiple of D + 1.  With one work-group per CU a stage's
// products take about 0.25 us, so the look-ahead has to cover the L2 and
// HBM latency under load (about 0.5-2 us) by itself: deeper rings and more
// register sets there, shallower ones where two work-groups share a CU.
// SPLITK > 1 (residual products): work-group k-slice ks of SPLITK stores its
// partial sums to a.split_out[ks][t][n]; resid_add_splits_kernel then adds
// the slices to the residual in order (no atomics: the sums do not depend on
// timing).
template <int EPI, int RBW, int TB, int D, int OCC, int SPLITK = 1, bool LO = false, int XA = 2>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OCC, OCC))) void gemm_deep_kernel(
    LinearArgs a, int n_wtiles, int n_ttiles) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int KS = 64;
    using C = GemmCfg<W_BF16, RBW, TB, KS, LO>;
    constexpr int KH = C::KH, NA = C::NA;
    constexpr int NX = XA + 1;                          // LDS ring depth
    static_assert(D == 1 || D == 3 || D == 7, "look-ahead");
    static_assert(XA >= 2 && XA <= 7, "activation look-ahead");
    static_assert(SPLITK == 1 || EPI == EPI_RESID, "k split: residual products only");
    __shared__ u32x4_t xs[NX * C::XF * 64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int total = n_wtiles * n_ttiles * SPLITK;
    const int b = blockIdx.x;
    const int tile = (total % 8 == 0) ? (b % 8) * (total / 8) + b / 8 : b;
    const int ks = tile % SPLITK;
    const int tt = (tile / SPLITK) % n_ttiles;
    const int nt = tile / (SPLITK * n_ttiles);
    const int nrb = a.N / 16;
    const int rb0 = nt * 4 * RBW + wave * RBW;
    const int t0 = tt * 16 * TB;
    const int nst_all = a.K / KS;
    const int sbeg = ks * (nst_all / SPLITK);          // this slice's stages [sbeg, nst)
    const int nst = sbeg + nst_all / SPLITK;

    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, (size_t)a.N * a.K * 2);
    const size_t xbytes = (size_t)(a.x.tiled ? (a.T + 15) / 16 * 16 : a.T) * a.x.ld * 2;
    const __amdgpu_buffer_rsrc_t rxh = make_rsrc(a.x.hi, xbytes);
    const __amdgpu_buffer_rsrc_t rxl = make_rsrc(LO ? a.x.lo : a.x.hi, xbytes);
    const int xst = a.x.tiled ? KS * 32 : KS * 2;     // bytes between stages
    // this wave's activation fragments f = wave*XW + u = (plane, token block, k half)
    int xoff[C::XW];
#pragma unroll
    for (int u = 0; u < C::XW; ++u) {
        const int f = wave * C::XW + u;
        const int tb = (f / KH) % TB, j = f % KH;
        xoff[u] = a.x.tiled ? ((t0 / 16 + tb) * (a.x.ld / 32) + j) * 1024 + lane * 16
                            : ((t0 + 16 * tb + r) * a.x.ld + 32 * j + 8 * g) * 2;
    }
    int woff[RBW];
#pragma unroll
    for (int i = 0; i < RBW; ++i) woff[i] = min(rb0 + i, nrb - 1) * 1024 + lane * 16;
    const int wstep = nrb * 1024;
    constexpr int NWL = RBW * NA;

    u32x4_t W[D + 1][RBW][NA];
    f32x4_t acc[RBW][TB];
#pragma unroll
    for (int i = 0; i < RBW; ++i)
#pragma unroll
        for (int j = 0; j < TB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // stage s's weights (clamped to the last stage: the loads past the end
    // keep the issue pattern, and so the wait counts, unchanged)
    auto issue_w = [&](int s, u32x4_t (&wn)[RBW][NA]) {
        const int sl = min(s, nst - 1);
#pragma unroll
        for (int j = 0; j < NA; ++j) {
            const int so = (NA * sl + j) * wstep;
#pragma unroll
            for (int i = 0; i < RBW; ++i) wn[i][j] = __builtin_amdgcn_raw_buffer_load_b128(rw, woff[i], so, 0);
        }
    };
    auto issue_x = [&](int s) {
        const int sl = min(s, nst - 1);
        u32x4_t *dst = xs + (size_t)((s % NX) * C::XF + wave * C::XW) * 64;
#pragma unroll
        for (int u = 0; u < C::XW; ++u) {
            const bool lo = (wave * C::XW + u) >= TB * KH;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(lo ? rxl : rxh,
                                                     (__attribute__((address_space(3))) void *)(dst + u * 64), 16,
                                                     xoff[u], sl * xst, 0, 0);
        }
    };
    // both k halves' activation fragments are read up front: the second
    // half's reads are in flight while the first half's products run
    static_assert(KH == 2, "two k halves per stage");
    auto compute = [&](int s, const u32x4_t (&wc)[RBW][NA]) {
        const u32x4_t *xb = xs + (size_t)(s % NX) * C::XF * 64;
        u32x4_t B[C::PL][2][TB];
#pragma unroll
        for (int pl = 0; pl < C::PL; ++pl)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) B[pl][j][tb] = xb[((pl * TB + tb) * KH + j) * 64 + lane];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int i = 0; i < RBW; ++i)
#pragma unroll
                    for (int pl = 0; pl < C::PL; ++pl)
                        acc[i][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wc[i][j]),
                                                                             __builtin_bit_cast(bf16x8_t, B[pl][j][tb]),
                                                                             acc[i][tb], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Stage t's iteration issues stage t + D's weights, then stage t + XA's
    // activations.  Loads return in issue order, so stage t may start once
    // no more are outstanding than were issued after the later of its two:
    // the weights (D < XA) are followed by one activation batch and D - 1
    // whole iterations, the activations by XA - 1 whole iterations.  The
    // prologue replays the iterations before the first stage, issuing only
    // the loads of stages >= sbeg, which leaves the same counts.
    constexpr int WAITN = D < XA ? C::XW + (D - 1) * (NWL + C::XW) : (XA - 1) * (NWL + C::XW);
    static_assert(WAITN + NWL + C::XW < 64, "loads in flight");
    constexpr int PRE = D > XA ? D : XA;
#pragma unroll
    for (int v = -PRE; v < 0; ++v) {
        if (v + D >= 0) issue_w(sbeg + v + D, W[(v + D) % (D + 1)]);
        if (v + XA >= 0) issue_x(sbeg + v + XA);
    }
    __builtin_amdgcn_sched_barrier(0);
    for (int s = sbeg; s < nst; s += D + 1) {
#pragma unroll
        for (int k = 0; k <= D; ++k) {
            wait_vm<WAITN>();
            wg_barrier();
            __builtin_amdgcn_sched_barrier(0);
            issue_w(s + k + D, W[(k + D) % (D + 1)]);
            issue_x(s + k + XA);
            __builtin_amdgcn_sched_barrier(0);
            compute(s + k, W[k]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    wait_vm<0>();

#pragma unroll
    for (int i = 0; i < RBW; ++i) {
        const int rb = rb0 + i;
        if (rb >= nrb) continue;
        if (EPI == EPI_SWIGLU && (i & 1)) continue;
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const int t = t0 + tb * 16 + r;
            if (t >= a.T) continue;
            if (SPLITK > 1)
                store4(a.split_out + ((size_t)ks * a.T + t) * a.N + rb * 16 + 4 * g, acc[i][tb]);
            else if (EPI == EPI_SWIGLU)
                epilogue4<EPI, false>(a, t, (rb >> 1) * 16 + 4 * g, acc[i][tb], acc[i + 1][tb]);
            else
                epilogue4<EPI, false>(a, t, rb * 16 + 4 * g, acc[i][tb], acc[i][tb]);
        }
    }
#endif
}

// Wide prefill product (bf16 weights, activations as hi + lo planes in
// operand-tiled order): a work-group of 8 waves in a 4 x 2 grid computes a
// (64 RBW)-row x (32 TBW)-token tile, wave (wr, wc) multiplying row blocks
// wr RBW .. + RBW by token blocks wc TBW .. + TBW.  Each 32-wide k stage's
// weights (4 RBW row-block fragments) and activations (2 TBW token blocks x
// 2 planes) go straight from global memory into an NX-deep LDS ring
// (buffer_load ... lds, each wave copying an equal run of fragments), NX - 1
// stages ahead, and every wave reads its operands out of LDS.  Each weight
// and activation byte crosses the load path once per work-group and feeds
// two (weights) or four (activations) waves: RBW = TBW = 4 (256 x 128) needs
// 128 bytes per MFMA, RBW = TBW = 2 (128 x 64) 256, where the deep kernel's
// 256 x 64 tile needs 192 and the products wait on that path.  The stage
// count K / 32 / SPLITK must be whole; SPLITK > 1 as the deep kernel.
template <int EPI, int SPLITK = 1, int NX = 4, int RBW = 4, int TBW = 4>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(
    NX * 4 * (RBW + TBW) <= 80 ? 4 : 2, NX * 4 * (RBW + TBW) <= 80 ? 4 : 2))) void
gemm_wide_kernel(LinearArgs a, int n_wtiles, int n_ttiles) {
    // (waves per SIMD: two work-groups share a CU when the ring's KB fit 80)
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int WF = 4 * RBW;           // weight fragments (1 KB) per stage
    constexpr int TBT = 2 * TBW;          // token blocks per tile
    constexpr int XF = 2 * TBT;           // activation fragments per stage (2 planes)
    constexpr int SF = WF + XF;
    constexpr int CPW = SF / 8;           // fragments each wave copies per stage
    static_assert(NX == 2 || NX == 4, "ring depth");
    static_assert(SF % 8 == 0 && WF % CPW == 0 && TBT % CPW == 0,
                  "each wave copies weights or one activation plane only");
    static_assert(SPLITK == 1 || EPI == EPI_RESID, "k split: residual products only");
    static_assert(EPI != EPI_SWIGLU || RBW % 2 == 0, "gate and up row blocks in pairs");
    __shared__ u32x4_t ring[NX * SF * 64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave >> 1, wc = wave & 1;
    const int r = lane & 15, g = lane >> 4;
    const int total = n_wtiles * n_ttiles * SPLITK;
    const int b = blockIdx.x;
    const int tile = (total % 8 == 0) ? (b % 8) * (total / 8) + b / 8 : b;
    const int ks = tile % SPLITK;
    const int tt = (tile / SPLITK) % n_ttiles;
    const int nt = tile / (SPLITK * n_ttiles);
    const int nrb = a.N / 16;
    const int rbt = nt * WF;              // the tile's first row block
    const int t0 = tt * TBT * 16;
    const int nst_all = a.K / 32;
    const int sbeg = ks * (nst_all / SPLITK), nst = sbeg + nst_all / SPLITK;

    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, (size_t)a.N * a.K * 2);
    const size_t xbytes = (size_t)((a.T + 15) / 16 * 16) * a.x.ld * 2;
    const __amdgpu_buffer_rsrc_t rxh = make_rsrc(a.x.hi, xbytes);
    const __amdgpu_buffer_rsrc_t rxl = make_rsrc(a.x.lo, xbytes);
    // this wave's copies: fragments f = CPW wave + u; f < WF is row block
    // rbt + f (clamped to the last row block: the epilogue skips rows past
    // N), else activation fragment f - WF = (plane, token block)
    const int f0 = CPW * wave;
    const bool wcopy = f0 < WF;
    const bool xlo = !wcopy && f0 - WF >= TBT;
    int off[CPW];
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
        const int f = f0 + u;
        off[u] = wcopy ? min(rbt + f, nrb - 1) * 1024 + lane * 16
                       : (t0 / 16 + (f - WF) % TBT) * (a.x.ld / 32) * 1024 + lane * 16;
    }
    const int sstep = wcopy ? nrb * 1024 : 1024;       // bytes between stages

    // stage s (clamped to the last: the loads past the end keep the issue
    // pattern, and so the wait counts, unchanged) into ring slot s % NX
    auto issue = [&](int s) {
        const int sl = min(s, nst - 1);
        u32x4_t *slot = ring + (size_t)(s % NX) * SF * 64;
#pragma unroll
        for (int u = 0; u < CPW; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wcopy ? rw : xlo ? rxl : rxh,
                                                     (__attribute__((address_space(3))) void *)(slot + (f0 + u) * 64),
                                                     16, off[u], sl * sstep, 0, 0);
    };

    f32x4_t acc[RBW][TBW];
#pragma unroll
    for (int i = 0; i < RBW; ++i)
#pragma unroll
        for (int j = 0; j < TBW; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // stage s needs its CPW copies landed: NX - 2 later stages may still be
    // in flight
#pragma unroll
    for (int k = 0; k < NX - 1; ++k) issue(sbeg + k);
    __builtin_amdgcn_sched_barrier(0);
    for (int s = sbeg; s < nst; ++s) {
        wait_vm<CPW * (NX - 2)>();
        wg_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue(s + NX - 1);
        __builtin_amdgcn_sched_barrier(0);
        const u32x4_t *slot = ring + (size_t)(s % NX) * SF * 64;
        u32x4_t A[RBW], B[2][TBW];
#pragma unroll
        for (int i = 0; i < RBW; ++i) A[i] = slot[(RBW * wr + i) * 64 + lane];
#pragma unroll
        for (int pl = 0; pl < 2; ++pl)
#pragma unroll
            for (int tb = 0; tb < TBW; ++tb) B[pl][tb] = slot[(WF + TBT * pl + TBW * wc + tb) * 64 + lane];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int tb = 0; tb < TBW; ++tb)
#pragma unroll
            for (int i = 0; i < RBW; ++i)
#pragma unroll
                for (int pl = 0; pl < 2; ++pl)
                    acc[i][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, A[i]),
                                                                         __builtin_bit_cast(bf16x8_t, B[pl][tb]),
                                                                         acc[i][tb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    // the ring's last copies must land before the work-group's LDS is released
    wait_vm<0>();

#pragma unroll
    for (int i = 0; i < RBW; ++i) {
        const int rb = rbt + RBW * wr + i;
        if (rb >= nrb) continue;
        if (EPI == EPI_SWIGLU && (i & 1)) continue;
#pragma unroll
        for (int tb = 0; tb < TBW; ++tb) {
            const int t = t0 + (TBW * wc + tb) * 16 + r;
            if (t >= a.T) continue;
            if (SPLITK > 1)
                store4(a.split_out + ((size_t)ks * a.T + t) * a.N + rb * 16 + 4 * g, acc[i][tb]);
            else if (EPI == EPI_SWIGLU)
                epilogue4<EPI, false>(a, t, (rb >> 1) * 16 + 4 * g, acc[i][tb], acc[i + 1][tb]);
            else
                epilogue4<EPI, false>(a, t, rb * 16 + 4 * g, acc[i][tb], acc[i][tb]);
        }
    }
#endif
}

// y[t][n] += the k slices' partial sums, slice 0 first
__global__ __launch_bounds__(256) void resid_add_splits_kernel(float *y, int ldy, const float *parts, int T, int N,
                                                               int nsplit) {
    const int n4 = N / 4;
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= (long)T * n4) return;
    const int t = (int)(i / n4), n = (int)(i % n4) * 4;
    f32x4_t v = *(const f32x4_t *)(parts + (size_t)t * N + n);
    for (int k = 1; k < nsplit; ++k) v += *(const f32x4_t *)(parts + ((size_t)k * T + t) * N + n);
    f32x4_t *o = (f32x4_t *)(y + (size_t)t * ldy + n);
    *o = *o + v;
}

__global__ __launch_bounds__(256) void rmsnorm_tiled_kernel(const float *x, int ldx, const int32_t *row_map,
                                                            const float *gain, int d, float eps, Act out);

// resid_add_splits_kernel and then rmsnorm_tiled_kernel of the updated rows
// in one pass: a work-group per row (the same row order), each thread adding
// the NS slices into its 8-value runs of the row (the same additions in the
// same order as resid_add_splits_kernel), storing them back and normalising
// them as rmsnorm_tiled_kernel does, so both outputs are those of the two
// kernels (N <= 8192: the runs stay in registers).  Every load of a thread
// is issued before the first addition.
template <int NS>
__global__ __launch_bounds__(256) void resid_add_norm_kernel(float *y, int ldy, const float *parts, int N,
                                                             const float *gain, float eps, Act out) {
    const int rows = gridDim.x, b = blockIdx.x;
    const int r = rows % 8 == 0 ? (b % 8) * (rows / 8) + b / 8 : b;
    float *yr = y + (size_t)r * ldy;
    constexpr int MAXV = 4;
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    f32x4_t v[MAXV][2], gn[MAXV][2], pk[MAXV][2][NS];
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int e = (threadIdx.x + 256 * i) * 8;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            v[i][h] = e < N ? *(const f32x4_t *)(yr + e + 4 * h) : z;
            gn[i][h] = e < N ? *(const f32x4_t *)(gain + e + 4 * h) : z;
#pragma unroll
            for (int k = 0; k < NS; ++k)
                pk[i][h][k] = e < N ? *(const f32x4_t *)(parts + ((size_t)k * rows + r) * N + e + 4 * h) : z;
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int e = (threadIdx.x + 256 * i) * 8;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            f32x4_t p = pk[i][h][0];
#pragma unroll
            for (int k = 1; k < NS; ++k) p += pk[i][h][k];
            v[i][h] = v[i][h] + p;
            if (e < N) *(f32x4_t *)(yr + e + 4 * h) = v[i][h];
        }
    }
#pragma unroll
    for (int i = 0; i < MAXV; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            ss += v[i][h][0] * v[i][h][0] + v[i][h][1] * v[i][h][1] + v[i][h][2] * v[i][h][2] +
                  v[i][h][3] * v[i][h][3];
    __shared__ float part[4];
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float inv = 1.0f / sqrtf((part[0] + part[1] + part[2] + part[3]) / (float)N + eps);
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int e = (threadIdx.x + 256 * i) * 8;
        if (e >= N) continue;
        const f32x4_t y0 = v[i][0] * inv * gn[i][0];
        const f32x4_t y1 = v[i][1] * inv * gn[i][1];
        u16x8_t hh, ll;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float yv = k < 4 ? y0[k] : y1[k - 4];
            hh[k] = f2bf(yv);
            ll[k] = f2bf(yv - bf2f(hh[k]));
        }
        const size_t o = act_idx(out, r, e);
        *(u16x8_t *)(out.hi + o) = hh;
        *(u16x8_t *)(out.lo + o) = ll;
    }
}

// After a residual product whose k was split into nsplit slices: the slices
// are added into y, with the post norm fused into that pass when asked for
// and possible (tiled output planes, rows of at most 8192 values).
static void finish_k_slices(const LinearArgs &a, int nsplit, hipStream_t s) {
    if (a.post.gain && a.post_done && g_tuning.post_norm != 0 && a.post.out.tiled && a.post.out.hi &&
        a.post.out.lo && a.N <= 8192 && a.N % 8 == 0 && (nsplit == 2 || nsplit == 4)) {
        if (nsplit == 2)
            UBD_LAUNCH(resid_add_norm_kernel<2>, dim3((unsigned)a.T), dim3(256), 0, s, a.y, a.ldy, a.split_out,
                       a.N, a.post.gain, a.post.eps, a.post.out);
        else
            UBD_LAUNCH(resid_add_norm_kernel<4>, dim3((unsigned)a.T), dim3(256), 0, s, a.y, a.ldy, a.split_out,
                       a.N, a.post.gain, a.post.eps, a.post.out);
        *a.post_done = true;
        return;
    }
    const long n = (long)a.T * (a.N / 4);
    UBD_LAUNCH(resid_add_splits_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.y, a.ldy,
               a.split_out, a.T, a.N, nsplit);
}

// false (nothing launched) unless each k slice's stage count is a multiple
// of D + 1 (and, split, the product is a residual one with scratch for the
// slices)
template <int EPI, int RBW, int TB, int D, int OCC, int SPLITK = 1, bool LO = false, int XA = 2>
static bool launch_gemm_deep(const LinearArgs &a, hipStream_t s) {
    const int nst = a.K / 64;
    if (a.K % 64 || nst % SPLITK || (nst / SPLITK) % (D + 1)) return false;
    if (SPLITK > 1 && (EPI != EPI_RESID || !a.split_out || a.N % 4)) return false;
    const int n_wtiles = (a.N + 64 * RBW - 1) / (64 * RBW);
    const int n_ttiles = (a.T + 16 * TB - 1) / (16 * TB);
    UBD_LAUNCH((gemm_deep_kernel<EPI, RBW, TB, D, OCC, SPLITK, LO, XA>), dim3(n_wtiles * n_ttiles * SPLITK),
                       dim3(256), 0, s, a, n_wtiles, n_ttiles);
    if (SPLITK > 1) finish_k_slices(a, SPLITK, s);
    return true;
}

// false (nothing launched) unless the operands are the tiled hi + lo planes
// and each k slice's stage count is whole (and, split, the product is a
// residual one with scratch for the slices)
template <int EPI, int SPLITK = 1, int NX = 4, int RBW = 4, int TBW = 4>
static bool launch_gemm_wide(const LinearArgs &a, hipStream_t s) {
    if (!a.x.tiled || !a.x.lo || a.K % 32 || (a.K / 32) % SPLITK) return false;
    if (SPLITK > 1 && (EPI != EPI_RESID || !a.split_out || a.N % 4)) return false;
    const int n_wtiles = (a.N + 64 * RBW - 1) / (64 * RBW);
    const int n_ttiles = (a.T + 32 * TBW - 1) / (32 * TBW);
    UBD_LAUNCH((gemm_wide_kernel<EPI, SPLITK, NX, RBW, TBW>), dim3(n_wtiles * n_ttiles * SPLITK), dim3(512), 0, s, a,
               n_wtiles, n_ttiles);
    if (SPLITK > 1) finish_k_slices(a, SPLITK, s);
    return true;
}

// wpd: stages of weight look-ahead (the tuning knob overrides it)
template <int WT, int EPI, int RBW, int TB, int SPLITK, bool LO = false>
static void launch_gemm_lds(const LinearArgs &a, hipStream_t s, int wpd = 1) {
    if constexpr (SPLITK > 1) {
        // the k slices go to scratch and are added in slice order: without
        // scratch (or for a product other than a residual one), no split
        if (EPI != EPI_RESID || !a.split_out || a.N % 4) {
            launch_gemm_lds<WT, EPI, RBW, TB, 1, LO>(a, s, wpd);
            return;
        }
    }
    const int n_wtiles = (a.N + 64 * RBW - 1) / (64 * RBW);
    const int n_ttiles = (a.T + 16 * TB - 1) / (16 * TB);
    const int total = n_wtiles * n_ttiles * SPLITK;
    if (g_tuning.gemm_wpd == 1 || g_tuning.gemm_wpd == 2) wpd = g_tuning.gemm_wpd;
    // 64-wide stages: the kernel then fits 2 waves per SIMD (two work-groups
    // per CU), which hides the LDS reads and barriers of one behind the other
    if (wpd == 2)
        UBD_LAUNCH((gemm_lds_kernel<WT, EPI, RBW, TB, SPLITK, 64, 2, LO>), dim3(total), dim3(256), 0, s, a,
                           n_wtiles, n_ttiles);
    else
        UBD_LAUNCH((gemm_lds_kernel<WT, EPI, RBW, TB, SPLITK, 64, 1, LO>), dim3(total), dim3(256), 0, s, a,
                           n_wtiles, n_ttiles);
    if (SPLITK > 1) finish_k_slices(a, SPLITK, s);
}

// Shape choice for the LDS-ring product: the largest tile (256 rows x 128
// tokens) when it yields enough work-groups for the 256 CUs, else narrower
// tiles; residual products may also split k (slices added in order).
// bf16 products over hi + lo activation planes (two products per
// fragment): twice the activation fragments per stage, so the tiles are at
// most 64 tokens wide.
template <int EPI>
static void launch_gemm_lds_shape_lo(const LinearArgs &a, hipStream_t s) {
    auto tiles = [&](int rbw, int tb) {
        return (long)((a.N + 64 * rbw - 1) / (64 * rbw)) * ((a.T + 16 * tb - 1) / (16 * tb));
    };
    constexpr int RS = EPI == EPI_RESID ? 2 : 1;
    // forced shapes for measurements and tests
    switch (g_tuning.gemm_shape) {
    case 1: launch_gemm_lds<W_BF16, EPI, 2, 4, 1, true>(a, s); return;
    case 3: launch_gemm_lds<W_BF16, EPI, 4, 4, 1, true>(a, s); return;
    case 5: if (EPI != EPI_SWIGLU) { launch_gemm_lds<W_BF16, EPI, 1, 4, 1, true>(a, s); return; } break;
    case 10: if (launch_gemm_deep<EPI, 2, 4, 3, 2, 1, true>(a, s)) return; break;
    case 14: if (launch_gemm_deep<EPI, 2, 4, 3, 2, RS, true>(a, s)) return; break;
    case 16: if (launch_gemm_deep<EPI, 4, 4, 1, 2, 1, true>(a, s)) return; break;
    case 18: if (launch_gemm_deep<EPI, 4, 4, 1, 2, RS, true>(a, s)) return; break;
    case 19: if (launch_gemm_deep<EPI, 4, 4, 1, 2, EPI == EPI_RESID ? 4 : 1, true>(a, s)) return; break;
    case 20: if (launch_gemm_deep<EPI, 2, 4, 3, 2, 1, true, 3>(a, s)) return; break;
    case 21: if (launch_gemm_wide<EPI, 1>(a, s)) return; break;
    case 22: if (launch_gemm_wide<EPI, EPI == EPI_RESID ? 4 : 1>(a, s)) return; break;
    case 23: if (launch_gemm_wide<EPI, 1, 2>(a, s)) return; break;
    case 24: if (launch_gemm_wide<EPI, 1, 4, 2, 2>(a, s)) return; break;
    case 25: if (launch_gemm_wide<EPI, EPI == EPI_RESID ? 2 : 1, 4, 2, 2>(a, s)) return; break;
    default: break;
    }
    if (EPI == EPI_RESID) {
        // k split over slices through scratch: forced (2 or 4), else in two
        // for long k (FFN down)
        constexpr int RS4 = EPI == EPI_RESID ? 4 : 1;
        if (g_tuning.gemm_split == 4 && launch_gemm_deep<EPI, 2, 4, 3, 2, RS4, true>(a, s)) return;
        if (g_tuning.gemm_split == 2 && launch_gemm_deep<EPI, 2, 4, 3, 2, RS, true>(a, s)) return;
        // long k (FFN down): the wide 256 x 128 tile in 4 k slices when that
        // gives a work-group per CU (8B shape at 512 tokens: 104 against 113
        // us), else the deep 256 x 64 tile (one stage of weight look-ahead) in
        // 4 slices (110.5 against 130.5 us for the 128 x 64 tile in 2)
        const long wide_tiles = (long)((a.N + 255) / 256) * ((a.T + 127) / 128);
        if (g_tuning.gemm_split == 0 && a.K >= 8192 && wide_tiles * 4 >= 256 && launch_gemm_wide<EPI, RS4>(a, s))
            return;
        if (g_tuning.gemm_split == 0 && a.K >= 8192 && tiles(4, 4) * 4 >= 256 &&
            launch_gemm_deep<EPI, 4, 4, 1, 2, RS4, true>(a, s))
            return;
        if (g_tuning.gemm_split == 0 && a.K >= 8192 && tiles(2, 4) * 2 >= 192 &&
            launch_gemm_deep<EPI, 2, 4, 3, 2, RS, true>(a, s))
            return;
        // short k (O): the wide kernel's 128 x 64 tile (8 waves of 32 x 32)
        // when there are >= 256 tiles (8B shape at 512 tokens: 40.9 against
        // 42.8 us), else the deep 128 x 64 tile with activations three stages
        // ahead in a 4-deep ring (40.7 against 43.8 us with two stages ahead;
        // deeper rings and more weight sets at one wave per SIMD measured no
        // better)
        if (tiles(2, 4) >= 256 && launch_gemm_wide<EPI, 1, 4, 2, 2>(a, s)) return;
        if (tiles(2, 4) >= 192 && launch_gemm_deep<EPI, 2, 4, 3, 2, 1, true, 3>(a, s)) return;
        launch_gemm_lds<W_BF16, EPI, 2, 4, 1, true>(a, s);
        return;
    }
    // QKV: the wide kernel's 128 x 64 tile (8 waves of 32 x 32) when there
    // are >= 256 tiles (8B shape at 512 tokens: 65.1 against 69.5 us), else
    // 64 x 64 tiles when they give >= 384 work-groups (69.9 us against 84.2
    // us for 256 x 64 and 72.0 us for the deep 128 x 64 tile)
    if (EPI == EPI_QKV && tiles(2, 4) >= 256 && launch_gemm_wide<EPI, 1, 4, 2, 2>(a, s)) return;
    if (EPI == EPI_QKV && tiles(1, 4) >= 384) {
        launch_gemm_lds<W_BF16, EPI, 1, 4, 1, true>(a, s);
        return;
    }
    // gate|up: the wide 256 x 128 tile with a 2-deep ring (two work-groups
    // per CU, so all of them resident at once) when there are >= 384 such
    // tiles (8B shape at 512 tokens: 195.9 against 205.4 us), else the deep
    // 256 x 64 tile with one stage of weight look-ahead in rotating register
    // sets when there are >= 2 work-groups per CU (203.1 us against 215.2 us
    // for the LDS-ring tile; the same tile on the O and down products is slower)
    if (EPI == EPI_SWIGLU && (long)((a.N + 255) / 256) * ((a.T + 127) / 128) >= 384 &&
        launch_gemm_wide<EPI, 1, 2>(a, s))
        return;
    if (EPI == EPI_SWIGLU && tiles(4, 4) >= 512 && launch_gemm_deep<EPI, 4, 4, 1, 2, 1, true>(a, s)) return;
    if (tiles(4, 4) >= 192)
        launch_gemm_lds<W_BF16, EPI, 4, 4, 1, true>(a, s);
    else
        launch_gemm_lds<W_BF16, EPI, 2, 4, 1, true>(a, s);
}

template <int WT, int EPI>
static void launch_gemm_lds_shape(const LinearArgs &a, hipStream_t s) {
    auto tiles = [&](int rbw, int tb) {
        return (long)((a.N + 64 * rbw - 1) / (64 * rbw)) * ((a.T + 16 * tb - 1) / (16 * tb));
    };
    if (WT == W_BF16 && ((g_tuning.prefill_lo >> a.prod) & 1)) {
        launch_gemm_lds_shape_lo<EPI>(a, s);
        return;
    }
    // forced shapes for measurements
    switch (g_tuning.gemm_shape) {
    case 1: launch_gemm_lds<WT, EPI, 2, 4, 1>(a, s); return;
    case 2: launch_gemm_lds<WT, EPI, 2, 8, 1>(a, s); return;
    case 3: launch_gemm_lds<WT, EPI, 4, 4, 1>(a, s); return;
    case 4: if (WT != W_Q8) { launch_gemm_lds<WT, EPI, WT == W_Q8 ? 2 : 4, 8, 1>(a, s); return; } break;
    case 5: if (EPI != EPI_SWIGLU) { launch_gemm_lds<WT, EPI, 1, 4, 1>(a, s); return; } break;
    case 6: if (EPI != EPI_SWIGLU) { launch_gemm_lds<WT, EPI, 1, 8, 1>(a, s); return; } break;
    case 7: if (WT == W_BF16 && launch_gemm_deep<EPI, 4, 8, 1, 1>(a, s)) return; break;
    case 8: if (WT == W_BF16 && launch_gemm_deep<EPI, 4, 8, 3, 1>(a, s)) return; break;
    case 9: if (WT == W_BF16 && launch_gemm_deep<EPI, 2, 8, 3, 2>(a, s)) return; break;
    case 10: if (WT == W_BF16 && launch_gemm_deep<EPI, 2, 4, 3, 2>(a, s)) return; break;
    case 11: if (WT == W_BF16 && launch_gemm_deep<EPI, 4, 4, 3, 2>(a, s)) return; break;
    case 12: if (WT == W_BF16 && launch_gemm_deep<EPI, 4, 16, 1, 1>(a, s)) return; break;
    case 13: if (WT == W_BF16 && launch_gemm_deep<EPI, 4, 4, 3, 2, EPI == EPI_RESID ? 2 : 1>(a, s)) return; break;
    case 14: if (WT == W_BF16 && launch_gemm_deep<EPI, 2, 4, 3, 2, EPI == EPI_RESID ? 2 : 1>(a, s)) return; break;
    case 15: if (WT == W_BF16 && launch_gemm_deep<EPI, 2, 8, 3, 2, EPI == EPI_RESID ? 2 : 1>(a, s)) return; break;
    default: break;
    }
    // bf16 products with enough tiles: the deep variant, weights three
    // stages ahead (measured at 512 tokens, 8B shape: O 44.4 -> 36.4 us,
    // FFN down 134.5 -> 108.5 us with 128 x 64 tiles; QKV 62.5 -> 58.2 us
    // with 128 x 128 tiles).  The wide gate|up tile keeps the kernel above.
    if (WT == W_BF16 && g_tuning.gemm_deep != 0) {
        // long-k residual products (FFN down): 128 x 128 tiles with k split in
        // two through scratch, slices added in order (down 93 -> 76 us)
        if (EPI == EPI_RESID && a.K >= 8192 && tiles(2, 8) * 2 >= 192 &&
            launch_gemm_deep<EPI, 2, 8, 3, 2, EPI == EPI_RESID ? 2 : 1>(a, s))
            return;
        if (EPI == EPI_RESID && tiles(2, 4) >= 192 && launch_gemm_deep<EPI, 2, 4, 3, 2>(a, s)) return;
        // QKV: 64 x 64 tiles of the LDS-ring kernel when they give >= 384
        // work-groups (52.4 against 55.9 us for the deep 128 x 128 tile at 512
        // tokens), else the deep kernel
        if (EPI == EPI_QKV && tiles(4, 8) < 192 && tiles(1, 4) >= 384) {
            launch_gemm_lds<WT, EPI, 1, 4, 1>(a, s);
            return;
        }
        if (EPI == EPI_QKV && tiles(4, 8) < 192 && tiles(2, 8) >= 192 && launch_gemm_deep<EPI, 2, 8, 3, 2>(a, s))
            return;
    }
    // residual products: 128 x 64 tiles, splitting k (slices through scratch,
    // added in order) only when there are too few tiles for the CUs
    if (EPI == EPI_RESID) {
        const long t = tiles(2, 4);
        if (g_tuning.gemm_split == 2) {
            launch_gemm_lds<WT, EPI, 2, 4, 2>(a, s);
            return;
        }
        if (g_tuning.gemm_split == 4) {
            launch_gemm_lds<WT, EPI, 2, 4, 4>(a, s);
            return;
        }
        // enough tiles: no split, weights two stages ahead (the narrow
        // tile leaves the registers for it; measured O 50.6 -> 44.5 us and
        // FFN down 143 -> 136 us at 512 tokens, 8B shape)
        if (t >= 192 || a.K < 1024)
            launch_gemm_lds<WT, EPI, 2, 4, 1>(a, s, 2);
        else if (t * 2 >= 192 || a.K < 2048)
            launch_gemm_lds<WT, EPI, 2, 4, 2>(a, s);
        else
            launch_gemm_lds<WT, EPI, 2, 4, 4>(a, s);
        return;
    }
    // wide products: 256 x 128 tiles (bf16) / 256 x 64 (q8_0: two activation
    // planes and the scale products); narrower ones 128 x 64
    if (WT == W_Q8 && tiles(4, 4) >= 192)
        launch_gemm_lds<WT, EPI, 4, 4, 1>(a, s);
    else if (WT != W_Q8 && tiles(4, 8) >= 192)
        launch_gemm_lds<WT, EPI, WT == W_Q8 ? 2 : 4, 8, 1>(a, s);
    else
        launch_gemm_lds<WT, EPI, 2, 4, 1>(a, s);
}

template <int WT, int EPI, int BT, int SPLITK>
static void launch_gemm(const LinearArgs &a, hipStream_t s) {
    const int n_wtiles = (a.N + 255) / 256;
    const int n_ttiles = (a.T + BT - 1) / BT;
    const int total = n_wtiles * n_ttiles * SPLITK;
    UBD_LAUNCH((gemm_kernel<WT, EPI, BT, SPLITK>), dim3(total), dim3(256), 0, s, a, n_wtiles, n_ttiles);
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
    if (g_tuning.gemm != 0) {
        launch_gemm_lds_shape<WT, EPI>(a, s);
        return true;
    }
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
    // k-split waves per work-group: about 4096 waves in flight, all resident
    int nw = blocks >= 768 ? 4 : blocks >= 384 ? 8 : 16;
    if (g_tuning.skinny_nw == 4 || g_tuning.skinny_nw == 8 || g_tuning.skinny_nw == 16) nw = g_tuning.skinny_nw;
    // gate|up pairs with 16 waves would spill registers to scratch
    if (EPI == EPI_SWIGLU && nw == 16) nw = 8;
    const bool norm = a.norm.x != nullptr;
    // activations of a 16-token block fit in LDS: the LDS-staged kernel
    // (hi and lo planes)
    const size_t ldsx = (size_t)4 * std::min(16, a.T) * a.K;
    if (ldsx <= LDSX_MAX_BYTES && g_tuning.ldsx != 0) {
        const size_t bytes = std::max(ldsx, (size_t)16 * 64 * 16 * 2);   // also holds the wave reduction
        LinearArgs la = a;
        la.early = g_tuning.ldsx_early;
#define UBD_LAUNCH_LDSX(NW_)                                                                                \
    do {                                                                                                    \
        if (norm)                                                                                           \
            UBD_LAUNCH((linear_ldsx_kernel<WT, EPI, NW_, true>), grid, dim3(64 * NW_), bytes, s, la); \
        else                                                                                                \
            UBD_LAUNCH((linear_ldsx_kernel<WT, EPI, NW_, false>), grid, dim3(64 * NW_), bytes, s, la); \
    } while (0)
        if (nw == 4)
            UBD_LAUNCH_LDSX(4);
        else if (nw == 8)
            UBD_LAUNCH_LDSX(8);
        else
            UBD_LAUNCH_LDSX(16);
#undef UBD_LAUNCH_LDSX
        return;
    }
    // the norm fused: its normalised rows staged in LDS when they fit (at
    // most NORM_TMAX rows of at most 8192 values, what norm_prologue holds),
    // else normalised on the fly (XN)
    const bool norm_lds = norm && a.T <= NORM_TMAX && a.K <= 8192 && (size_t)4 * a.T * a.K <= LDSX_MAX_BYTES;
    const size_t lds = norm_lds ? (size_t)4 * a.T * a.K : 0;
    if (a.T > 2 && g_tuning.small_rb != 0) {
        // several tokens: 4 row blocks per work-group share each activation
        // fragment when that still gives >= 256 work-groups per token block;
        // narrower products use 2 row blocks or (residual products) split k
        const int nrb = a.N / 16;
        if (nrb % 4 == 0 && nrb / 4 >= 256) {
            dim3 g4(nrb / 4, grid.y);
            const int nw4 = nrb / 4 >= 768 ? 4 : 8;
            if (nw4 == 4 && norm)
                UBD_LAUNCH((linear_small_kernel<WT, EPI, 4, false, 4, 1, true>), g4, dim3(256), 0, s, a);
            else if (nw4 == 4)
                UBD_LAUNCH((linear_small_kernel<WT, EPI, 4, false, 4, 1>), g4, dim3(256), 0, s, a);
            else if (norm)
                UBD_LAUNCH((linear_small_kernel<WT, EPI, 8, false, 4, 1, true>), g4, dim3(512), 0, s, a);
            else
                UBD_LAUNCH((linear_small_kernel<WT, EPI, 8, false, 4, 1>), g4, dim3(512), 0, s, a);
            return;
        }
        // narrower products that cannot split k (QKV): 2 row blocks, 16 waves
        if (nrb % 2 == 0 && nrb / 2 >= 192) {
            dim3 g2(nrb / 2, grid.y);
            if (norm)
                UBD_LAUNCH((linear_small_kernel<WT, EPI, 16, false, 2, 1, true>), g2, dim3(1024), 0, s, a);
            else
                UBD_LAUNCH((linear_small_kernel<WT, EPI, 16, false, 2, 1>), g2, dim3(1024), 0, s, a);
            return;
        }
        constexpr int KSPLIT = EPI == EPI_RESID ? 4 : 1;
        if (KSPLIT > 1 && !norm && nrb % 4 == 0 && (a.K / WT_<WT>::KSTEP) % 32 == 0) {
            dim3 g4(nrb / 4, grid.y, KSPLIT);
            UBD_LAUNCH((linear_small_kernel<WT, EPI, 8, false, 4, KSPLIT>), g4, dim3(512), 0, s, a);
            return;
        }
    }
#define UBD_LAUNCH_SMALL(NW_)                                                                                \
    do {                                                                                                     \
        if (norm_lds)                                                                                        \
            UBD_LAUNCH((linear_small_kernel<WT, EPI, NW_, true, RB, 1>), grid, dim3(64 * NW_), lds, s, a);     \
        else if (norm)                                                                                       \
            UBD_LAUNCH((linear_small_kernel<WT, EPI, NW_, false, RB, 1, true>), grid, dim3(64 * NW_), 0, s, a); \
        else                                                                                                 \
            UBD_LAUNCH((linear_small_kernel<WT, EPI, NW_, false, RB, 1>), grid, dim3(64 * NW_), 0, s, a);     \
    } while (0)
    if (nw == 4)
        UBD_LAUNCH_SMALL(4);
    else if (nw == 8)
        UBD_LAUNCH_SMALL(8);
    else
        UBD_LAUNCH_SMALL(16);
#undef UBD_LAUNCH_SMALL
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

// mirrors the dispatch: try_gemm takes bf16 / q8_0 products of >= 64 tokens
// with K a multiple of 64, and runs an LDS-ring kernel unless the
// register-staged one is selected
bool linear_reads_tiled(const LinearArgs &a) {
    return g_tuning.act_tiled != 0 && g_tuning.gemm != 0 && (a.wtype == W_BF16 || a.wtype == W_Q8) && a.T >= 64 &&
           a.K % 64 == 0 && !(a.epi == EPI_SWIGLU && a.N % 32) && a.norm.x == nullptr && a.N > 0;
}

bool linear_norm_fits(int T, int K) {
    // one- and few-token products (the LDS-staged kernel normalises up to 16
    // rows into its stage; the other few-token kernel stages up to
    // NORM_TMAX rows or normalises on the fly)
    (void)K;
    return T >= 1 && T <= 16;
}

bool launch_linear(const LinearArgs &a, hipStream_t s) {
    if (a.T <= 0 || a.N <= 0) return true;
    if (a.norm.x && !linear_norm_fits(a.T, a.K)) return false;
    switch (a.wtype) {
    case W_F32: launch_linear_wt<W_F32>(a, s); break;
    case W_BF16: launch_linear_wt<W_BF16>(a, s); break;
    case W_Q8: launch_linear_wt<W_Q8>(a, s); break;
    default: return false;
    }
    return true;
}

// ------------------------------------------------------------ embedding
__global__ __launch_bounds__(256) void embed_kernel(int wtype, const void *table, const uint16_t *scales,
                                                    int d, TokInfo ti, float *x, int32_t *cell_pos,
                                                    uint32_t *cell_seq, int n_cells, const double *inv_freq,
                                                    int half_dim, float2 *rope_cs) {
    const int t = blockIdx.x;
    if (threadIdx.x < half_dim) {
        double sn, cs;
        sincos((double)ti.pos[t] * inv_freq[threadIdx.x], &sn, &cs);
        rope_cs[(size_t)t * half_dim + threadIdx.x] = make_float2((float)cs, (float)sn);
    }
    const size_t row = (size_t)ti.token[t];
    float *xo = x + (size_t)t * d;
    for (int e = threadIdx.x * 4; e < d; e += 1024) {      // d is a multiple of 16
        f32x4_t v;
        if (wtype == W_F32) {
            v = *(const f32x4_t *)((const float *)table + row * d + e);
        } else if (wtype == W_BF16) {
            const u16x4_t h = *(const u16x4_t *)((const uint16_t *)table + row * d + e);
            v = f32x4_t{bf2f(h[0]), bf2f(h[1]), bf2f(h[2]), bf2f(h[3])};
        } else {
            const uint32_t q = *(const uint32_t *)((const int8_t *)table + row * d + e);
            const float sc = h2f(scales[row * (d / 32) + e / 32]);
            v = f32x4_t{(float)(int8_t)q, (float)(int8_t)(q >> 8), (float)(int8_t)(q >> 16),
                        (float)(int8_t)(q >> 24)} * sc;
        }
        *(f32x4_t *)(xo + e) = v;
    }
    if (threadIdx.x == 0) cell_pos[(size_t)ti.stream[t] * n_cells + ti.cell[t]] = ti.pos[t];
    if (threadIdx.x < ti.n_seq_words) {
        const int w = threadIdx.x;
        cell_seq[((size_t)ti.stream[t] * ti.n_seq_words + w) * n_cells + ti.cell[t]] =
            ti.seqw[(size_t)t * ti.n_seq_words + w];
    }
}

void launch_embed(int wtype, const void *table, const uint16_t *scales, int d, const TokInfo &ti, int T,
                  float *x, int32_t *cell_pos, uint32_t *cell_seq, int n_cells, const double *inv_freq,
                  int half_dim, float2 *rope_cs, hipStream_t s) {
    if (T <= 0) return;
    UBD_LAUNCH(embed_kernel, dim3(T), dim3(256), 0, s, wtype, table, scales, d, ti, x, cell_pos,
                       cell_seq, n_cells, inv_freq, half_dim, rope_cs);
}

// -------------------------------------------------------------- RMSNorm
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float *x, int ldx, const int32_t *row_map,
                                                      const float *gain, int d, float eps, Act out) {
    // d is a multiple of 16: every thread handles whole float4s, loads issued
    // together before the reduction
    const int r = blockIdx.x;
    const int src = row_map ? row_map[r] : r;
    const float *xr = x + (size_t)src * ldx;
    constexpr int MAXV = 8;                  // float4 per thread held in registers (d <= 8192)
    f32x4_t v[MAXV];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int e = (threadIdx.x + 256 * i) * 4;
        v[i] = e < d ? *(const f32x4_t *)(xr + e) : f32x4_t{0.f, 0.f, 0.f, 0.f};
        ss += v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] + v[i][3] * v[i][3];
    }
    for (int e = (threadIdx.x + 256 * MAXV) * 4; e < d; e += 1024) {
        const f32x4_t w = *(const f32x4_t *)(xr + e);
        ss += w[0] * w[0] + w[1] * w[1] + w[2] * w[2] + w[3] * w[3];
    }
    __shared__ float part[4];
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float inv = 1.0f / sqrtf((part[0] + part[1] + part[2] + part[3]) / (float)d + eps);
    const size_t ob = (size_t)r * out.ld;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int e = (threadIdx.x + 256 * i) * 4;
        if (e < d) {
            const f32x4_t y = v[i] * inv * *(const f32x4_t *)(gain + e);
#pragma unroll
            for (int k = 0; k < 4; ++k) store_act(out, ob + e + k, y[k]);
        }
    }
    for (int e = (threadIdx.x + 256 * MAXV) * 4; e < d; e += 1024) {
        const f32x4_t y = *(const f32x4_t *)(xr + e) * inv * *(const f32x4_t *)(gain + e);
#pragma unroll
        for (int k = 0; k < 4; ++k) store_act(out, ob + e + k, y[k]);
    }
}

// RMSNorm of one row into tiled HILO activations (d a multiple of 32): every
// thread owns 8-value runs, each one lane's 16 bytes of an operand tile, so
// the two planes take one 16-byte store per run.
// Work-group b takes row (b % 8) * (rows / 8) + b / 8 when rows is a multiple
// of 8: work-groups go to the 8 XCDs in turn, so each XCD writes whole
// 16-row blocks of the tiled output, whose 128-byte lines interleave 8 rows.
__global__ __launch_bounds__(256) void rmsnorm_tiled_kernel(const float *x, int ldx, const int32_t *row_map,
                                                            const float *gain, int d, float eps, Act out) {
    const int rows = gridDim.x, b = blockIdx.x;
    const int r = rows % 8 == 0 ? (b % 8) * (rows / 8) + b / 8 : b;
    const float *xr = x + (size_t)(row_map ? row_map[r] : r) * ldx;
    constexpr int MAXV = 4;                  // 8-value runs per thread held in registers (d <= 8192)
    // the row and its gains are loaded together, so the gains' round trip
    // hides under the row's
    f32x4_t v[MAXV][2], gn[MAXV][2];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int e = (threadIdx.x + 256 * i) * 8;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            v[i][h] = e < d ? *(const f32x4_t *)(xr + e + 4 * h) : f32x4_t{0.f, 0.f, 0.f, 0.f};
            gn[i][h] = e < d ? *(const f32x4_t *)(gain + e + 4 * h) : f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
#pragma unroll
    for (int i = 0; i < MAXV; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            ss += v[i][h][0] * v[i][h][0] + v[i][h][1] * v[i][h][1] + v[i][h][2] * v[i][h][2] +
                  v[i][h][3] * v[i][h][3];
    for (int e = (threadIdx.x + 256 * MAXV) * 8; e < d; e += 2048)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const f32x4_t w = *(const f32x4_t *)(xr + e + 4 * h);
            ss += w[0] * w[0] + w[1] * w[1] + w[2] * w[2] + w[3] * w[3];
        }
    __shared__ float part[4];
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float inv = 1.0f / sqrtf((part[0] + part[1] + part[2] + part[3]) / (float)d + eps);
    auto put = [&](int e, f32x4_t a0, f32x4_t a1, f32x4_t g0, f32x4_t g1) {
        const f32x4_t y0 = a0 * inv * g0;
        const f32x4_t y1 = a1 * inv * g1;
        u16x8_t hh, ll;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float y = k < 4 ? y0[k] : y1[k - 4];
            hh[k] = f2bf(y);
            ll[k] = f2bf(y - bf2f(hh[k]));
        }
        const size_t o = act_idx(out, r, e);
        *(u16x8_t *)(out.hi + o) = hh;
        *(u16x8_t *)(out.lo + o) = ll;
    };
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int e = (threadIdx.x + 256 * i) * 8;
        if (e < d) put(e, v[i][0], v[i][1], gn[i][0], gn[i][1]);
    }
    for (int e = (threadIdx.x + 256 * MAXV) * 8; e < d; e += 2048)
        put(e, *(const f32x4_t *)(xr + e), *(const f32x4_t *)(xr + e + 4), *(const f32x4_t *)(gain + e),
            *(const f32x4_t *)(gain + e + 4));
}

void launch_rmsnorm(const float *x, int ldx, const int32_t *row_map, int rows, const float *gain, int d,
                    float eps, const Act &out, hipStream_t s) {
    if (rows <= 0) return;
    if (out.tiled) {
        UBD_LAUNCH(rmsnorm_tiled_kernel, dim3(rows), dim3(256), 0, s, x, ldx, row_map, gain, d, eps, out);
        return;
    }
    UBD_LAUNCH(rmsnorm_kernel, dim3(rows), dim3(256), 0, s, x, ldx, row_map, gain, d, eps, out);
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
    __shared__ int cpos[SUB];
    __shared__ uint32_t cseq[MAX_SEQ_WORDS][SUB];
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
    const size_t vbase = ((size_t)st * a.n_head_kv + g) * HD * a.n_cells;  // 32-cell tiles
    const int32_t *cp = a.cell_pos + (size_t)st * a.n_cells;
    const uint32_t *cs = a.cell_seq + (size_t)st * a.n_seq_words * a.n_cells;

    for (int sub = cbeg; sub < cend; sub += SUB) {
        const int ns = min(SUB, cend - sub);
        __syncthreads();
        for (int e = tid; e < SUB * HD; e += 256) {
            const int c = e / HD, d = e % HD;
            Kt[d][c] = c < ns ? load_kv(a.k_cache, a.type_k, kbase + (size_t)(sub + c) * HD + d) : 0.f;
        }
        for (int e = tid; e < SUB * HD; e += 256) {
            const int d = e / SUB, c = e % SUB;
            Vt[d][c] = c < ns ? load_kv(a.v_cache, a.type_v, vbase + v_off(HD, d, (size_t)(sub + c))) : 0.f;
        }
        if (tid < SUB) cpos[tid] = tid < ns ? cp[sub + tid] : -1;
        for (int e = tid; e < a.n_seq_words * SUB; e += 256) {
            const int w = e / SUB, c = e % SUB;
            cseq[w][c] = c < ns ? cs[(size_t)w * a.n_cells + sub + c] : 0u;
        }
        __syncthreads();
        for (int e = tid; e < R * SUB; e += 256) {
            const int row = e / SUB, c = e % SUB;
            float sv = -INFINITY;
            const int rs = rseq[row];
            if (c < ns && ((cseq[rs >> 5][c] >> (rs & 31)) & 1u) && cpos[c] >= 0 && cpos[c] <= rpos[row]) {
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
        store_act(a.out, act_idx(a.out, t, h * HD + d), o * invL);
    }
}

template <int HD>
static void launch_attention_hd(const AttnArgs &a, hipStream_t s) {
    dim3 grid(a.max_chunks, a.n_tiles, a.n_head_kv);
    UBD_LAUNCH(attn_partial_kernel<HD>, grid, dim3(256), 0, s, a);
    UBD_LAUNCH(attn_combine_kernel<HD>, dim3(a.T * a.n_head), dim3(128), 0, s, a);
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
// the cell order {4g..4g+3, 16+4g..16+4g+3}, which the V tile supplies as
// one contiguous 16-byte run per lane.  The product is taken as
// O^T = V^T P^T, so lane (row r, group g) also holds O[r][dims 4g+i] of
// each 16-dim block: a row's softmax state (m, l), its rescale factor and
// its outputs all stay in the row's lanes.  Online softmax per row; SPLIT
// writes the range's (m, l, O) for a combine pass, otherwise O / l is stored.
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

// Buffer resources over this (stream, KV head)'s K rows, V^T tiles, the
// stream's cell positions and sequence words, and this lane's byte offsets
// into them, fixed across steps: a step adds only a scalar offset, so its
// loads need no per-lane address arithmetic.
template <int HD> struct KVSrc {
    __amdgpu_buffer_rsrc_t k, v, pos, seq;
    int ko, vo, po, so;         // so: this lane's row's sequence-mask word
};

// One 32-cell step of K (two 16-cell MFMA A blocks), V^T (the P*V B
// fragments) and the cells' (pos, seq).
template <int HD> struct KVStep {
    static constexpr int KK = HD / 32, DB = HD / 16;
    f16x8_t k[2][KK];
    f16x8_t v[DB];
    int4 p[2], s[2];
};

// NT: the K/V codes are loaded non-temporally (streams read once per step:
// long split scans), else through the caches (prefill tiles re-read them).
template <typename T, bool NT>
__device__ __forceinline__ T kv_ld(const T *p) {
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

template <int HD, bool NT>
__device__ __forceinline__ void kv_step_load(KVStep<HD> &b, const KVSrc<HD> &src, int c0) {
    constexpr int KK = HD / 32, DB = HD / 16;
    constexpr int aux = NT ? 2 : 0;     // non-temporal
    const int cu = __builtin_amdgcn_readfirstlane(c0);
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) {
        const int cb = cu + 16 * b2;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            b.k[b2][kk] = __builtin_bit_cast(
                f16x8_t, __builtin_amdgcn_raw_buffer_load_b128(src.k, src.ko + 64 * kk, cb * HD * 2, aux));
        b.p[b2] = __builtin_bit_cast(int4, __builtin_amdgcn_raw_buffer_load_b128(src.pos, src.po, cb * 4, 0));
        b.s[b2] = __builtin_bit_cast(int4, __builtin_amdgcn_raw_buffer_load_b128(src.seq, src.so, cb * 4, 0));
    }
    // c0 is a multiple of 32: the step's V is the contiguous tile c0 / 32,
    // and this lane's B fragment of dims 16 db + r is slots 8g .. 8g+7
#pragma unroll
    for (int db = 0; db < DB; ++db)
        b.v[db] = __builtin_bit_cast(f16x8_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                  src.v, src.vo + db * 16 * 32 * 2, (cu >> 5) * HD * 32 * 2, aux));
}

// The MFMA attention works in base 2: the query carries log2(e) / sqrt(hd),
// so scores, the running max m and the chunk maxima are log2-scaled and every
// exponential is one native 2^x (exp(s - m) = 2^(log2e s - log2e m)).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Max and sum over the four 16-lane rows holding one query row's values
// (lanes r, r + 16, r + 32, r + 48): the row pairs swap through the gfx950
// permlane swaps (vector ALU, no LDS round trip).  Each returns a lane's
// value and its partner's, 16 then 32 lanes apart; max and + commute, so
// every lane of a row gets the same result.
__device__ __forceinline__ float row_max(float v) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row_sum(float v) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Scores of the step's 32 cells for the wave's 16 rows, mask, online-softmax
// update of (m, l) and O += P V.
template <int HD>
__device__ __forceinline__ void kv_step_compute(const KVStep<HD> &b, int c0, int cend, const f16x8_t *qh,
                                                const f16x8_t *ql, bool row_ok, int rbit, int rpos, int g,
                                                float &m, float &l, f32x4_t *O) {
    constexpr int KK = HD / 32, DB = HD / 16;
    f32x4_t S[2];
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(b.k[b2][kk], qh[kk], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(b.k[b2][kk], ql[kk], acc, 0, 0, 0);
        }
        const int cc = c0 + 16 * b2 + 4 * g;
        const int pp[4] = {b.p[b2].x, b.p[b2].y, b.p[b2].z, b.p[b2].w};
        const int ss[4] = {b.s[b2].x, b.s[b2].y, b.s[b2].z, b.s[b2].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool vis = row_ok && cc + i < cend && (((uint32_t)ss[i] >> rbit) & 1u) && pp[i] >= 0 &&
                             pp[i] <= rpos;
            acc[i] = vis ? acc[i] : -INFINITY;
        }
        S[b2] = acc;
    }
    const float mx = row_max(fmaxf(fmaxf(fmaxf(S[0][0], S[0][1]), fmaxf(S[0][2], S[0][3])),
                                   fmaxf(fmaxf(S[1][0], S[1][1]), fmaxf(S[1][2], S[1][3]))));
    const float m_new = fmaxf(m, mx);
    const float alpha = (m_new == -INFINITY) ? 1.f : exp2_fast(m - m_new);
    float ps = 0.f;
    f16x8_t ph, pl;
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float sv = S[b2][i];
            const float p = sv == -INFINITY ? 0.f : exp2_fast(sv - m_new);
            ps += p;
            const _Float16 h = (_Float16)p;
            ph[4 * b2 + i] = h;
            pl[4 * b2 + i] = (_Float16)(p - (float)h);
        }
    l = l * alpha + row_sum(ps);
    m = m_new;
    // V^T fragments as A and P^T as B: the output holds this lane's row r
    // (dims 16 db + 4g + i), whose rescale factor the lane already has
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        f32x4_t o = O[db] * alpha;
        o = __builtin_amdgcn_mfma_f32_16x16x32_f16(b.v[db], ph, o, 0, 0, 0);
        o = __builtin_amdgcn_mfma_f32_16x16x32_f16(b.v[db], pl, o, 0, 0, 0);
        O[db] = o;
    }
}

// ----- q8_0 K/V: the int8 codes enter bf16 MFMAs exactly; q and P are
// split hi + lo in bf16 (whose exponent range keeps small P * scale
// products out of subnormals).  K scales (one per cell and 32-dim block)
// multiply the score partial of each block; V scales are folded into P per
// 32-dim block of V.
template <int HD> struct KVSrcQ8 {
    const int8_t *K, *Vt;
    const uint16_t *ks, *vs;    // [HD/32][cells] f16 scales of this (stream, KV head)
    const int32_t *cpos;
    const uint32_t *cseq;       // the sequence-mask word of this lane's row
    int n_cells, r, g;
};

template <int HD> struct KVStepQ8 {
    static constexpr int KK = HD / 32, DB = HD / 16;
    u32x2_t k[2][KK];   // codes: cell cb + r, dims 32 kk + 8g .. + 8
    u32x2_t ksc[2][KK]; // K scales of the D rows: cells cb + 4g .. + 4, block kk
    u32x2_t v[DB];      // codes: dim 16 db + r, slots 8g .. 8g + 8
    u32x2_t vsc[KK][2]; // V scales of the P columns: cells c0 + 4g .., c0 + 16 + 4g .., block b
    int4 p[2], s[2];
};

template <int HD, bool NT>
__device__ __forceinline__ void kv_step_load_q8(KVStepQ8<HD> &b, const KVSrcQ8<HD> &src, int c0) {
    constexpr int KK = HD / 32, DB = HD / 16;
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) {
        const int cb = c0 + 16 * b2;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            b.k[b2][kk] = kv_ld<u32x2_t, NT>((const u32x2_t *)(src.K + (size_t)(cb + src.r) * HD + 32 * kk + 8 * src.g));
            b.ksc[b2][kk] = *(const u32x2_t *)(src.ks + (size_t)kk * src.n_cells + cb + 4 * src.g);
        }
        b.p[b2] = *(const int4 *)(src.cpos + cb + 4 * src.g);
        b.s[b2] = *(const int4 *)(src.cseq + cb + 4 * src.g);
    }
    const int8_t *vt = src.Vt + (size_t)(c0 >> 5) * HD * 32 + src.r * 32 + 8 * src.g;
#pragma unroll
    for (int db = 0; db < DB; ++db) b.v[db] = kv_ld<u32x2_t, NT>((const u32x2_t *)(vt + db * 16 * 32));
#pragma unroll
    for (int kb = 0; kb < KK; ++kb) {
        b.vsc[kb][0] = *(const u32x2_t *)(src.vs + (size_t)kb * src.n_cells + c0 + 4 * src.g);
        b.vsc[kb][1] = *(const u32x2_t *)(src.vs + (size_t)kb * src.n_cells + c0 + 16 + 4 * src.g);
    }
}

__device__ __forceinline__ float h2f_lo(uint32_t w) { return h2f((uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float h2f_hi(uint32_t w) { return h2f((uint16_t)(w >> 16)); }

template <int HD>
__device__ __forceinline__ void kv_step_compute_q8(const KVStepQ8<HD> &b, int c0, int cend, const bf16x8_t *qh,
                                                   const bf16x8_t *ql, bool row_ok, int rbit, int rpos, int g,
                                                   float &m, float &l, f32x4_t *O) {
    constexpr int KK = HD / 32;
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    f32x4_t S[2];
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) {
        f32x4_t acc = z;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const bf16x8_t A = i8x8_to_bf16(b.k[b2][kk][0], b.k[b2][kk][1]);
            f32x4_t d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, qh[kk], z, 0, 0, 0);
            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, ql[kk], d, 0, 0, 0);
            const f32x4_t sc = {h2f_lo(b.ksc[b2][kk][0]), h2f_hi(b.ksc[b2][kk][0]), h2f_lo(b.ksc[b2][kk][1]),
                                h2f_hi(b.ksc[b2][kk][1])};
            acc += sc * d;
        }
        const int cc = c0 + 16 * b2 + 4 * g;
        const int pp[4] = {b.p[b2].x, b.p[b2].y, b.p[b2].z, b.p[b2].w};
        const int ss[4] = {b.s[b2].x, b.s[b2].y, b.s[b2].z, b.s[b2].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool vis = row_ok && cc + i < cend && (((uint32_t)ss[i] >> rbit) & 1u) && pp[i] >= 0 &&
                             pp[i] <= rpos;
            acc[i] = vis ? acc[i] : -INFINITY;
        }
        S[b2] = acc;
    }
    const float mx = row_max(fmaxf(fmaxf(fmaxf(S[0][0], S[0][1]), fmaxf(S[0][2], S[0][3])),
                                   fmaxf(fmaxf(S[1][0], S[1][1]), fmaxf(S[1][2], S[1][3]))));
    const float m_new = fmaxf(m, mx);
    const float alpha = (m_new == -INFINITY) ? 1.f : exp2_fast(m - m_new);
    float pv[8];
    float ps = 0.f;
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float sv = S[b2][i];
            const float p = sv == -INFINITY ? 0.f : exp2_fast(sv - m_new);
            ps += p;
            pv[4 * b2 + i] = p;
        }
    l = l * alpha + row_sum(ps);
    m = m_new;
#pragma unroll
    for (int kb = 0; kb < KK; ++kb) {
        // P of this lane's 8 cells times their V scales of dim block kb
        f32x8_t x;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t w = b.vsc[kb][e >> 2][(e & 3) >> 1];
            x[e] = pv[e] * ((e & 1) ? h2f_hi(w) : h2f_lo(w));
        }
        const bf16x8_t Ph = __builtin_convertvector(x, bf16x8_t);
        const bf16x8_t Pl = __builtin_convertvector(x - __builtin_convertvector(Ph, f32x8_t), bf16x8_t);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const int db = 2 * kb + h2;
            const bf16x8_t Vf = i8x8_to_bf16(b.v[db][0], b.v[db][1]);
            f32x4_t o = O[db] * alpha;
            o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Vf, Ph, o, 0, 0, 0);
            o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Vf, Pl, o, 0, 0, 0);
            O[db] = o;
        }
    }
}

// NW > 1 (no split): a work-group of NW waves per (tile, KV head); wave w
// scans the w-th of NW runs of 32-cell steps of the tile's cells, and the
// waves merge their (m, l, O) through LDS, each finishing the dim blocks
// db = w, w + NW, ...  The grid is (KV head, tile) with the tiles in reverse
// order, so the longest causal scans start first (prefill: two waves).
// (For decode steps with short scans, four waves merged this way measured
// slower than the split pass and its combine kernel: each wave's steps wait
// on their loads one after another.)
// NT: K/V codes loaded non-temporally (long split scans).
template <int HD, bool SPLIT, bool KQ, int NW = 1, bool NT = false>
__global__ __launch_bounds__(NW * 64) void attn_mfma_kernel(AttnArgs a) {
    static_assert(!(SPLIT && NW > 1), "the multi-wave mode merges in the work-group");
    constexpr int KK = HD / 32, DB = HD / 16;
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    const int wv = NW > 1 ? (int)(threadIdx.x >> 6) : 0;
    const int chunk = NW > 1 ? 0 : blockIdx.x;
    const int blk = NW > 1 ? a.n_tiles - 1 - (int)blockIdx.y : (int)blockIdx.y;
    const int grp = NW > 1 ? blockIdx.x : blockIdx.z;
    const int t0 = a.tok.tiles[blk * 4 + 0], nt = a.tok.tiles[blk * 4 + 1];
    const int st = a.tok.tiles[blk * 4 + 2], nscan = a.tok.tiles[blk * 4 + 3];
    const int G = a.n_head / a.n_head_kv;
    const int R = nt * G;
    const int NC = a.chunk_cells;
    int cbeg = 0, cend = nscan;
    if (SPLIT) {
        cbeg = chunk * NC;
        if (cbeg >= nscan) {
            // past this tile's cells: an empty partial (m = -inf, l = 0), so
            // the merge can take every launched chunk without looking up
            // the tile's scan length
            if ((lane >> 4) == 0 && (lane & 15) < R) {
                const int row = lane & 15;
                float *ml = a.part_ml +
                            (((size_t)(t0 + row / G) * a.n_head + grp * G + row % G) * a.max_chunks + chunk) * 2;
                ml[0] = -INFINITY;
                ml[1] = 0.f;
            }
            return;
        }
        cend = min(nscan, cbeg + NC);
    }
    if (NW > 1) {
        const int per = (nscan + 32 * NW - 1) / (32 * NW) * 32;   // a multiple of 32 cells
        cbeg = min(nscan, wv * per);
        cend = min(nscan, cbeg + per);
    }
    const float scale = 1.44269504088896341f / sqrtf((float)HD);   // log2(e) / sqrt(hd)
    // this lane's query row (S^T layout: row = r)
    const bool row_ok = r < R;
    const int rt = t0 + (row_ok ? r / G : 0), rh = grp * G + (row_ok ? r % G : 0);
    const int rpos = a.tok.pos[rt], rseq = a.tok.seq[rt], rbit = rseq & 31;
    // every lane loads a valid row (rows past R read row 0) and zeroes it
    // afterwards, so the loads are unconditional and issued together
    const float *qrow = a.q + (size_t)rt * a.n_head * HD + rh * HD + 8 * g;
    const float qs = row_ok ? scale : 0.f;
    float4 qv[KK][2];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        qv[kk][0] = *(const float4 *)(qrow + 32 * kk);
        qv[kk][1] = *(const float4 *)(qrow + 32 * kk + 4);
    }
    float m = -INFINITY, l = 0.f;
    f32x4_t O[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) O[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int32_t *cpos = a.cell_pos + (size_t)st * a.n_cells;
    const uint32_t *cseq = a.cell_seq + ((size_t)st * a.n_seq_words + (rseq >> 5)) * a.n_cells;
    const size_t hbase = (size_t)st * a.n_head_kv + grp;

    // Two register sets: the loads of the next 32-cell step are in flight
    // while the current one is computed.  Past the range the load repeats
    // the current step's cells (in bounds, served by the cache) and the
    // compute masks every cell, so the loop has no data-dependent branch.
    // (The scheduling fences keep the next step's score MFMAs, which do not
    // depend on the softmax state, from being hoisted above the current
    // step and forcing an early wait on loads just issued.)
    if constexpr (!KQ) {
        f16x8_t qh[KK], ql[KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const float e8[8] = {qv[kk][0].x, qv[kk][0].y, qv[kk][0].z, qv[kk][0].w,
                                 qv[kk][1].x, qv[kk][1].y, qv[kk][1].z, qv[kk][1].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = e8[e] * qs;
                const _Float16 h = (_Float16)v;
                qh[kk][e] = h;
                ql[kk][e] = (_Float16)(v - (float)h);
            }
        }
        const _Float16 *K = (const _Float16 *)a.k_cache + hbase * a.n_cells * HD;
        const _Float16 *Vt = (const _Float16 *)a.v_cache + hbase * a.n_cells * HD;
        const size_t kvb = (size_t)a.n_cells * HD * 2;
        const KVSrc<HD> src{make_rsrc(K, kvb),
                            make_rsrc(Vt, kvb),
                            make_rsrc(cpos, (size_t)a.n_cells * 4),
                            make_rsrc(a.cell_seq + (size_t)st * a.n_seq_words * a.n_cells,
                                      (size_t)a.n_seq_words * a.n_cells * 4),
                            (r * HD + 8 * g) * 2,
                            (r * 32 + 8 * g) * 2,
                            16 * g,
                            ((rseq >> 5) * a.n_cells + 4 * g) * 4};
        KVStep<HD> A, B;
        if (cbeg < cend) kv_step_load<HD, NT>(A, src, cbeg);
        for (int c0 = cbeg; c0 < cend; c0 += 64) {
            const int c1 = c0 + 32, c2 = c0 + 64;
            kv_step_load<HD, NT>(B, src, c1 < cend ? c1 : c0);
            __builtin_amdgcn_sched_barrier(0);
            kv_step_compute(A, c0, cend, qh, ql, row_ok, rbit, rpos, g, m, l, O);
            __builtin_amdgcn_sched_barrier(0);
            kv_step_load<HD, NT>(A, src, c2 < cend ? c2 : c0);
            __builtin_amdgcn_sched_barrier(0);
            kv_step_compute(B, c1, cend, qh, ql, row_ok, rbit, rpos, g, m, l, O);
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        bf16x8_t qh[KK], ql[KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const float e8[8] = {qv[kk][0].x, qv[kk][0].y, qv[kk][0].z, qv[kk][0].w,
                                 qv[kk][1].x, qv[kk][1].y, qv[kk][1].z, qv[kk][1].w};
            f32x8_t v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = e8[e] * qs;
            qh[kk] = __builtin_convertvector(v, bf16x8_t);
            ql[kk] = __builtin_convertvector(v - __builtin_convertvector(qh[kk], f32x8_t), bf16x8_t);
        }
        const int8_t *K = (const int8_t *)a.k_cache + hbase * a.n_cells * HD;
        const int8_t *Vt = (const int8_t *)a.v_cache + hbase * a.n_cells * HD;
        const uint16_t *ks = (const uint16_t *)((const int8_t *)a.k_cache + a.layer_elems) + hbase * KK * a.n_cells;
        const uint16_t *vs = (const uint16_t *)((const int8_t *)a.v_cache + a.layer_elems) + hbase * KK * a.n_cells;
        const KVSrcQ8<HD> src{K, Vt, ks, vs, cpos, cseq, a.n_cells, r, g};
        KVStepQ8<HD> A, B;
        if (cbeg < cend) kv_step_load_q8<HD, NT>(A, src, cbeg);
        for (int c0 = cbeg; c0 < cend; c0 += 64) {
            const int c1 = c0 + 32, c2 = c0 + 64;
            kv_step_load_q8<HD, NT>(B, src, c1 < cend ? c1 : c0);
            __builtin_amdgcn_sched_barrier(0);
            kv_step_compute_q8(A, c0, cend, qh, ql, row_ok, rbit, rpos, g, m, l, O);
            __builtin_amdgcn_sched_barrier(0);
            kv_step_load_q8<HD, NT>(A, src, c2 < cend ? c2 : c0);
            __builtin_amdgcn_sched_barrier(0);
            kv_step_compute_q8(B, c1, cend, qh, ql, row_ok, rbit, rpos, g, m, l, O);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // O: lane (row r, group g) holds dims 16 db + 4g + i of its row, and
    // the row's (m, l)
    if constexpr (NW > 1) {
        // every wave publishes its (m, l) per row and its O; each lane then
        // weights the NW partials of its row by exp2(m_w - M) and finishes
        // its wave's dim blocks
        __shared__ float pm[NW][16], pl[NW][16];
        __shared__ f32x4_t po[NW][DB][64];
        if (g == 0) {
            pm[wv][r] = m;
            pl[wv][r] = l;
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) po[wv][db][lane] = O[db];
        __syncthreads();
        float wgt[NW];
        float M = -INFINITY, L = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, pm[w][r]);
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float mw = pm[w][r];
            wgt[w] = mw == -INFINITY ? 0.f : exp2_fast(mw - M);
            L += wgt[w] * pl[w][r];
        }
        if (!row_ok) return;
#pragma unroll
        for (int db = wv; db < DB; db += NW) {
            f32x4_t o = po[0][db][lane] * wgt[0];
#pragma unroll
            for (int w = 1; w < NW; ++w) o += po[w][db][lane] * wgt[w];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                store_act(a.out, act_idx(a.out, rt, rh * HD + 16 * db + 4 * g + i), L > 0.f ? o[i] / L : 0.f);
        }
        return;
    }
    if (!row_ok) return;
    if (!SPLIT) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                store_act(a.out, act_idx(a.out, rt, rh * HD + 16 * db + 4 * g + i), l > 0.f ? O[db][i] / l : 0.f);
        return;
    }
    // split: publish this chunk's (m, l, O) for the combine pass
    const size_t pidx = ((size_t)rt * a.n_head + rh) * a.max_chunks + chunk;
    if (g == 0) {
        a.part_ml[pidx * 2] = m;
        a.part_ml[pidx * 2 + 1] = l;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) *(f32x4_t *)(a.part_o + pidx * HD + 16 * db + 4 * g) = O[db];
}

// Merge the chunks of one (token, head): weights exp(m_c - M) computed
// lane-parallel over chunks, then every dim sums its chunks with the loads
// of a 64-chunk pass issued together.  Every launched chunk has a partial
// (empty ones m = -inf, weight 0, their O never read into the sum).
template <int HD>
__global__ __launch_bounds__(64) void attn_merge_kernel(AttnArgs a) {
    const int t = blockIdx.x / a.n_head, h = blockIdx.x % a.n_head;
    const int lane = threadIdx.x;
    const int nch = a.n_chunks_launch;
    const float *ml = a.part_ml + ((size_t)t * a.n_head + h) * a.max_chunks * 2;
    const float *po = a.part_o + ((size_t)t * a.n_head + h) * a.max_chunks * HD;
    float M = -INFINITY;
    for (int c = lane; c < nch; c += 64) M = fmaxf(M, ml[2 * c]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    float L = 0.f;
    constexpr int DPL = (HD + 63) / 64;
    float o[DPL];
#pragma unroll
    for (int j = 0; j < DPL; ++j) o[j] = 0.f;
    for (int c0 = 0; c0 < nch; c0 += 64) {
        const int c = c0 + lane;
        float wgt = 0.f;
        if (c < nch) {
            const float mc = ml[2 * c];
            wgt = mc == -INFINITY ? 0.f : exp2_fast(mc - M);
            L += wgt * ml[2 * c + 1];
        }
        const int n = min(64, nch - c0);
        for (int k = 0; k < n; k += 8) {
            float w8[8], v8[8][DPL];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                w8[u] = __shfl(wgt, min(k + u, 63), 64);
#pragma unroll
                for (int j = 0; j < DPL; ++j) {
                    const int d = lane + 64 * j;
                    v8[u][j] = (k + u < n && d < HD) ? po[(size_t)(c0 + k + u) * HD + d] : 0.f;
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int j = 0; j < DPL; ++j) o[j] += (k + u < n && w8[u] != 0.f) ? w8[u] * v8[u][j] : 0.f;
        }
    }
    L = wave_sum(L);
    const float invL = L > 0.f ? 1.0f / L : 0.f;
#pragma unroll
    for (int j = 0; j < DPL; ++j) {
        const int d = lane + 64 * j;
        if (d < HD) store_act(a.out, act_idx(a.out, t, h * HD + d), o[j] * invL);
    }
}

template <int HD>
static void launch_attention_mfma_hd(const AttnArgs &a, hipStream_t s) {
    const bool q8 = a.type_k == KV_Q8;
    if (a.split) {
        dim3 grid((unsigned)a.n_chunks_launch, a.n_tiles, a.n_head_kv);
        if (q8 && a.kv_nt)
            UBD_LAUNCH((attn_mfma_kernel<HD, true, true, 1, true>), grid, dim3(64), 0, s, a);
        else if (q8)
            UBD_LAUNCH((attn_mfma_kernel<HD, true, true>), grid, dim3(64), 0, s, a);
        else if (a.kv_nt)
            UBD_LAUNCH((attn_mfma_kernel<HD, true, false, 1, true>), grid, dim3(64), 0, s, a);
        else
            UBD_LAUNCH((attn_mfma_kernel<HD, true, false>), grid, dim3(64), 0, s, a);
        UBD_LAUNCH((attn_merge_kernel<HD>), dim3(a.T * a.n_head), dim3(64), 0, s, a);
    } else if (a.waves == 2) {
        dim3 grid(a.n_head_kv, a.n_tiles);
        if (q8)
            UBD_LAUNCH((attn_mfma_kernel<HD, false, true, 2>), grid, dim3(128), 0, s, a);
        else
            UBD_LAUNCH((attn_mfma_kernel<HD, false, false, 2>), grid, dim3(128), 0, s, a);
    } else {
        dim3 grid(1, a.n_tiles, a.n_head_kv);
        if (q8)
            UBD_LAUNCH((attn_mfma_kernel<HD, false, true>), grid, dim3(64), 0, s, a);
        else
            UBD_LAUNCH((attn_mfma_kernel<HD, false, false>), grid, dim3(64), 0, s, a);
    }
}

bool attn_mfma_ok(int type_k, int type_v, int head_dim, int n_gqa) {
    return ((type_k == KV_F16 && type_v == KV_F16) || (type_k == KV_Q8 && type_v == KV_Q8)) && n_gqa <= 16 &&
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
// ARGMAX_BLOCKS work-groups per row each reduce a slice; the last one to
// finish (counted with an atomic) reduces the slices' winners and re-arms
// the counter.  Ties go to the lowest index.
__device__ __forceinline__ void better(float &bv, int &bi, float v, int i) {
    if (v > bv || (v == bv && i < bi)) {
        bv = v;
        bi = i;
    }
}

__device__ __forceinline__ void block_best(float &bv, int &bi) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        better(bv, bi, ov, oi);
    }
    __shared__ float sv[4];
    __shared__ int si[4];
    if ((threadIdx.x & 63) == 0) {
        sv[threadIdx.x >> 6] = bv;
        si[threadIdx.x >> 6] = bi;
    }
    __syncthreads();
    bv = sv[0];
    bi = si[0];
    for (int w = 1; w < 4; ++w) better(bv, bi, sv[w], si[w]);
}

// out2 (may be null): a second copy of each row's pick (chained greedy
// steps: the next step's token-table slot on the device).
__global__ __launch_bounds__(256) void argmax_kernel(const float *logits, int ld, const int32_t *rows, int n,
                                                     int32_t *out, float *pv, int32_t *pi, int32_t *counter,
                                                     int32_t *out2) {
    const int row = blockIdx.y, b = blockIdx.x, nb = gridDim.x;
    const float *z = logits + (size_t)(rows ? rows[row] : row) * ld;
    const int chunk = ((n + nb - 1) / nb + 3) & ~3;
    const int beg = b * chunk, end = min(n, beg + chunk);
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int i = beg + threadIdx.x * 4; i < end; i += 1024) {     // n is a multiple of 16
        const f32x4_t v = *(const f32x4_t *)(z + i);
#pragma unroll
        for (int k = 0; k < 4; ++k) better(bv, bi, v[k], i + k);
    }
    block_best(bv, bi);
    if (!counter) {
        // two-pass form: argmax_final_kernel reduces the slices
        if (threadIdx.x == 0) {
            pv[row * nb + b] = bv;
            pi[row * nb + b] = bi;
        }
        return;
    }
    __shared__ int last;
    if (threadIdx.x == 0) {
        pv[row * nb + b] = bv;
        pi[row * nb + b] = bi;
        __threadfence();
        last = atomicAdd(counter + row, 1) == nb - 1;
    }
    __syncthreads();
    if (!last) return;
    __threadfence();
    bv = -INFINITY;
    bi = 0x7fffffff;
    for (int k = threadIdx.x; k < nb; k += blockDim.x)
        better(bv, bi, __hip_atomic_load(pv + row * nb + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
               __hip_atomic_load(pi + row * nb + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    block_best(bv, bi);
    if (threadIdx.x == 0) {
        const int32_t pick = bi == 0x7fffffff ? 0 : bi;
        out[row] = pick;
        if (out2) out2[row] = pick;
        counter[row] = 0;
    }
}

// Second pass of the two-pass argmax: one work-group per row reduces the
// row's slice winners in slice order (ties: the lowest index).
__global__ __launch_bounds__(256) void argmax_final_kernel(const float *pv, const int32_t *pi, int nb,
                                                           int32_t *out) {
    const int row = blockIdx.x;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int k = threadIdx.x; k < nb; k += blockDim.x) better(bv, bi, pv[row * nb + k], pi[row * nb + k]);
    block_best(bv, bi);
    if (threadIdx.x == 0) out[row] = bi == 0x7fffffff ? 0 : bi;
}

void launch_argmax_two_pass(const float *logits, int ld, int n_rows, int n, int32_t *out, float *pv, int32_t *pi,
                            hipStream_t s) {
    if (n_rows <= 0) return;
    UBD_LAUNCH(argmax_kernel, dim3(ARGMAX_BLOCKS, n_rows), dim3(256), 0, s, logits, ld,
                       (const int32_t *)nullptr, n, out, pv, pi, (int32_t *)nullptr, (int32_t *)nullptr);
    UBD_LAUNCH(argmax_final_kernel, dim3(n_rows), dim3(256), 0, s, pv, pi, ARGMAX_BLOCKS, out);
}

void launch_argmax(const float *logits, int ld, const int32_t *rows, int n_rows, int n, int32_t *out,
                   const ArgmaxWork &w, hipStream_t s, int32_t *out2) {
    if (n_rows <= 0) return;
    UBD_LAUNCH(argmax_kernel, dim3(ARGMAX_BLOCKS, n_rows), dim3(256), 0, s, logits, ld, rows, n, out, w.pv,
                       w.pi, w.counter, out2);
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
    const size_t tile = idx >> 6;                   // k-step-major: tile = s * (N/16) + rb
    const int lane = (int)(idx & 63);
    const int NB = a.N / 16;
    const int rb = (int)(tile % NB), s = (int)(tile / NB);
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
        // codes stored as q + 128 (sign bit flipped): the decode products
        // take them as offset bytes directly (q8w_to_bf16 flips them back)
        const int8_t *row = (const int8_t *)a.src[si].data + (size_t)sr * a.K;
        *(u32x2_t *)dst = *(const u32x2_t *)(row + 64 * s + 8 * g) ^ 0x80808080u;
        *(u32x2_t *)(dst + 8) = *(const u32x2_t *)(row + 64 * s + 32 + 8 * g) ^ 0x80808080u;
    }
}

// q8_0 scales: per 16-row block rb and 64-wide k-step s (blocks 2s, 2s+1),
// 32 f16 values ordered [g][h][i] = row 4g + i of block 2s + h, so the
// scales a lane group g needs for one k-step are one 16-byte run.
__global__ __launch_bounds__(256) void relayout_scales_kernel(RelayoutArgs a) {
    const int KB = a.K / 32, KP = KB / 2;
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t total = (size_t)a.N * KB;
    if (idx >= total) return;
    const int i = (int)(idx & 3), h = (int)((idx >> 2) & 1), g = (int)((idx >> 3) & 3);
    const size_t rest = idx >> 5;
    const int p = (int)(rest % KP), rb = (int)(rest / KP);
    int si, sr;
    map_row(a, rb * 16 + 4 * g + i, &si, &sr);
    a.dst_scales[idx] = a.src[si].scales[(size_t)sr * KB + 2 * p + h];
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
    UBD_LAUNCH(relayout_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
    if (wtype == W_Q8) {
        const size_t ts = (size_t)a.N * (K / 32);
        UBD_LAUNCH(relayout_scales_kernel, dim3((unsigned)((ts + 255) / 256)), dim3(256), 0, s, a);
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
            idx = ((size_t)stream * n_head_kv + head) * n_cells * hd + v_off(hd, d, c);
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
    UBD_LAUNCH(kv_store_kernel, grid, dim3(256), 0, s, src, src_type, n, cells, cache, type,
                       (int)transposed, stream, n_head_kv, hd, n_cells);
}

__global__ __launch_bounds__(256) void kv_load_kernel(const void *cache, int type, int transposed, int stream,
                                                      int cell0, int n, int n_head_kv, int hd, int n_cells,
                                                      size_t layer_elems, float *out) {
    const int W = n_head_kv * hd;
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)n * W) return;
    const int p = (int)(idx / W), j = (int)(idx % W);
    const int head = j / hd, d = j % hd;
    const size_t c = (size_t)cell0 + p;
    size_t src;
    if (transposed)
        src = ((size_t)stream * n_head_kv + head) * n_cells * hd + v_off(hd, d, c);
    else
        src = (((size_t)stream * n_head_kv + head) * n_cells + c) * hd + d;
    if (type == KV_Q8) {
        const uint16_t *sc = (const uint16_t *)((const int8_t *)cache + layer_elems);
        const size_t si = (((size_t)stream * n_head_kv + head) * (hd / 32) + d / 32) * n_cells + c;
        out[idx] = h2f(sc[si]) * (float)((const int8_t *)cache)[src];
        return;
    }
    out[idx] = load_kv(cache, type, src);
}

void launch_kv_load(const void *cache, int type, bool transposed, int stream, int cell0, int n, int n_head_kv,
                    int hd, int n_cells, size_t layer_elems, float *out, hipStream_t s) {
    if (n <= 0) return;
    const size_t total = (size_t)n * n_head_kv * hd;
    UBD_LAUNCH(kv_load_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, cache, type,
                       (int)transposed, stream, cell0, n, n_head_kv, hd, n_cells, layer_elems, out);
}

// Defrag moves: one thread per stored value.  The tmp rows are [n][Hk*hd]
// values of the cache's own type; q8_0 scales follow in a second plane
// [n][Hk*hd/32] after the codes (256-byte aligned).
template <typename E>
__global__ __launch_bounds__(256) void kv_move_kernel(void *cache, int transposed, int stream,
                                                      const int32_t *cells, int n, int n_head_kv, int hd,
                                                      int n_cells, size_t layer_elems, int q8, void *tmp,
                                                      int to_tmp) {
    const int W = n_head_kv * hd;
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)n * W) return;
    const int m = (int)(idx / W), j = (int)(idx % W);
    const int head = j / hd, d = j % hd;
    const size_t c = (size_t)cells[m];
    const size_t ci = transposed ? ((size_t)stream * n_head_kv + head) * n_cells * hd + v_off(hd, d, c)
                                 : (((size_t)stream * n_head_kv + head) * n_cells + c) * hd + d;
    E *cp = (E *)cache;
    E *tp = (E *)tmp;
    if (to_tmp)
        tp[idx] = cp[ci];
    else
        cp[ci] = tp[idx];
    if (q8 && d % 32 == 0) {
        uint16_t *sc = (uint16_t *)((int8_t *)cache + layer_elems);
        uint16_t *ts = (uint16_t *)((int8_t *)tmp + ((size_t)n * W + 255) / 256 * 256);
        const size_t si = (((size_t)stream * n_head_kv + head) * (hd / 32) + d / 32) * n_cells + c;
        const size_t ti = (size_t)m * (W / 32) + j / 32;
        if (to_tmp)
            ts[ti] = sc[si];
        else
            sc[si] = ts[ti];
    }
}

size_t kv_move_tmp_bytes(int type, int n, int n_head_kv, int hd) {
    const size_t vals = (size_t)n * n_head_kv * hd;
    if (type == KV_Q8) return (vals + 255) / 256 * 256 + vals / 32 * 2;
    return vals * (type == KV_F32 ? 4 : 2);
}

void launch_kv_move(void *cache, int type, bool transposed, int stream, const int32_t *cells, int n,
                    int n_head_kv, int hd, int n_cells, size_t layer_elems, void *tmp, bool to_tmp,
                    hipStream_t s) {
    if (n <= 0) return;
    const size_t total = (size_t)n * n_head_kv * hd;
    const dim3 grid((unsigned)((total + 255) / 256));
    if (type == KV_F32)
        UBD_LAUNCH(kv_move_kernel<uint32_t>, grid, dim3(256), 0, s, cache, (int)transposed, stream, cells,
                           n, n_head_kv, hd, n_cells, layer_elems, 0, tmp, (int)to_tmp);
    else if (type == KV_F16)
        UBD_LAUNCH(kv_move_kernel<uint16_t>, grid, dim3(256), 0, s, cache, (int)transposed, stream, cells,
                           n, n_head_kv, hd, n_cells, layer_elems, 0, tmp, (int)to_tmp);
    else
        UBD_LAUNCH(kv_move_kernel<uint8_t>, grid, dim3(256), 0, s, cache, (int)transposed, stream, cells,
                           n, n_head_kv, hd, n_cells, layer_elems, 1, tmp, (int)to_tmp);
}

// One thread per 34-byte block; the block start is 2-byte aligned.
__global__ __launch_bounds__(256) void q8_blocks_split_kernel(const uint16_t *blocks, size_t nb, int8_t *codes,
                                                              uint16_t *scales) {
    const size_t b = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nb) return;
    const uint16_t *p = blocks + b * 17;
    scales[b] = p[0];
    uint16_t *c = (uint16_t *)(codes + b * 32);
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = p[1 + i];
}

void launch_q8_blocks_split(const void *blocks, size_t n_blocks, int8_t *codes, uint16_t *scales,
                            hipStream_t s) {
    if (n_blocks == 0) return;
    UBD_LAUNCH(q8_blocks_split_kernel, dim3((unsigned)((n_blocks + 255) / 256)), dim3(256), 0, s,
                       (const uint16_t *)blocks, n_blocks, codes, scales);
}

__global__ __launch_bounds__(256) void f16_to_f32_kernel(const uint16_t *src, size_t n, float *dst) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = h2f(src[i]);
}

void launch_f16_to_f32(const uint16_t *src, size_t n, float *dst, hipStream_t s) {
    if (n == 0) return;
    UBD_LAUNCH(f16_to_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, n, dst);
}

// q8_0 quantisation of KV rows into their cells: 32 lanes per 32-value
// block (8 blocks per work-group).  All arithmetic is single float32
// operations with IEEE rounding (amax / 127, 1 / d, x * (1 / d)), then
// rounding to nearest with halves away from zero, so the codes follow from
// the inputs alone.
__global__ __launch_bounds__(256) void kv_quant_kernel(const void *src, int src_type, int ld, int n,
                                                       const int32_t *cells, const int32_t *streams, int stream,
                                                       void *cache, int is_v, int n_head_kv, int hd, int n_cells,
                                                       size_t layer_elems) {
    const int nb = n_head_kv * hd / 32;                  // blocks per row
    const size_t blk = ((size_t)blockIdx.x * 256 + threadIdx.x) / 32;
    const int j = threadIdx.x & 31;
    if (blk >= (size_t)n * nb) return;                   // whole 32-lane groups leave together
    const int r = (int)(blk / nb), b = (int)(blk % nb);
    const int head = b / (hd / 32), hb = b % (hd / 32), d = hb * 32 + j;
    const size_t si = (size_t)r * ld + head * hd + d;
    const float x = src_type == KV_F32 ? ((const float *)src)[si] : h2f(((const uint16_t *)src)[si]);
    float amax = fabsf(x);
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 32));
    const float dsc = __fdiv_rn(amax, 127.0f);
    const float inv = dsc > 0.f ? __fdiv_rn(1.0f, dsc) : 0.f;
    const float q = roundf(__fmul_rn(x, inv));
    const int st = streams ? streams[r] : stream;
    const size_t c = (size_t)cells[r];
    const size_t hb0 = (size_t)st * n_head_kv + head;
    int8_t *codes = (int8_t *)cache;
    if (is_v)
        codes[hb0 * n_cells * hd + v_off(hd, d, c)] = (int8_t)q;
    else
        codes[(hb0 * n_cells + c) * hd + d] = (int8_t)q;
    if (j == 0) ((uint16_t *)(codes + layer_elems))[(hb0 * (hd / 32) + hb) * n_cells + c] = f2h(dsc);
}

void launch_kv_quant(const void *src, int src_type, int ld, int n, const int32_t *cells, const int32_t *streams,
                     int stream, void *cache, bool is_v, int n_head_kv, int hd, int n_cells, size_t layer_elems,
                     hipStream_t s) {
    if (n <= 0) return;
    const size_t threads = (size_t)n * n_head_kv * hd;   // one lane per value
    UBD_LAUNCH(kv_quant_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, src, src_type, ld,
                       n, cells, streams, stream, cache, (int)is_v, n_head_kv, hd, n_cells, layer_elems);
}

}  // namespace ubd
