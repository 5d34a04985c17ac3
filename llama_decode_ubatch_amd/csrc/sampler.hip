// Sampler chain on one logits row (engine page, Steps 14-16, "Sampler
// chain": penalties, then the top-k / top-p / min-p cut-offs, then
// temperature, then the choice of one token).  One work-group of 1024
// threads per call:
//   1. radix select (3 passes of 11/11/10 bits over an order-preserving key
//      of each logit) of the (top_k + n_hist)-th largest logit T;
//   2. every token with logit >= T goes into an LDS candidate list: this
//      holds the post-penalty top-k, because penalties change only history
//      tokens and at most n_hist of those rank above any other token;
//   3. history tokens get their penalty (and join the list if they were
//      below T);
//   4. bitonic sort by (logit descending, id ascending), keep top_k;
//   5. top-p, min-p, temperature and the draw with u use block scans of the
//      softmax weights in that order.
#include "kernels.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

namespace ubd {

namespace {

constexpr int TPB = 1024;
constexpr int CAP = 4096;             // candidate list capacity (LDS)
static_assert(SAMPLER_KMAX + 2 * SAMPLER_HMAX <= CAP, "fallback list plus history must fit");
static_assert(SAMPLER_HMAX <= TPB && SAMPLER_KMAX <= 2 * TPB, "one thread per history token; scans of 2 per thread");

__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t b = __float_as_uint(f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// inclusive prefix sums of v[0 .. n), n <= 2 * TPB, by every thread
template <typename T>
__device__ void block_scan(T *v, int n) {
    for (int off = 1; off < n; off <<= 1) {
        const int i0 = threadIdx.x, i1 = threadIdx.x + TPB;
        const T a0 = (i0 < n && i0 >= off) ? v[i0 - off] : T(0);
        const T a1 = (i1 < n && i1 >= off) ? v[i1 - off] : T(0);
        __syncthreads();
        if (i0 < n && i0 >= off) v[i0] += a0;
        if (i1 < n && i1 >= off) v[i1] += a1;
        __syncthreads();
    }
}

__device__ __forceinline__ bool before(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

__global__ __launch_bounds__(TPB) void sampler_kernel(SamplerArgs a) {
    __shared__ uint32_t hist[2048];
    __shared__ float cv[CAP];
    __shared__ int ci[CAP];
    __shared__ float w[2048];
    __shared__ int s_n, s_overflow, s_cut;
    __shared__ uint32_t s_digit, s_rank;
    const int tid = threadIdx.x;
    const int V = a.n_vocab;
    const int need = min(V, a.top_k + a.n_hist);

    // 1. radix select of the need-th largest key
    uint32_t prefix = 0, pmask = 0, rank = (uint32_t)need;
    for (int pass = 0; pass < 3; ++pass) {
        const int sh = pass == 0 ? 21 : pass == 1 ? 10 : 0;
        const int nb = pass == 2 ? 1024 : 2048;
        for (int b = tid; b < 2048; b += TPB) hist[b] = 0;
        __syncthreads();
        for (int i = tid; i < V; i += TPB) {
            const uint32_t k = order_key(a.logits[i]);
            if ((k & pmask) == prefix) atomicAdd(&hist[(k >> sh) & (nb - 1)], 1u);
        }
        __syncthreads();
        // counts from the top bin down, then the bin where the rank falls
        for (int j = tid; j < nb; j += TPB) w[j] = (float)hist[nb - 1 - j];   // counts < 2^24: exact
        __syncthreads();
        block_scan(w, nb);
        for (int j = tid; j < nb; j += TPB) {
            const float above = j ? w[j - 1] : 0.f;
            if (w[j] >= (float)rank && above < (float)rank) {
                s_digit = (uint32_t)(nb - 1 - j);
                s_rank = rank - (uint32_t)above;
            }
        }
        __syncthreads();
        prefix |= s_digit << sh;
        pmask |= (uint32_t)(nb - 1) << sh;
        rank = s_rank;
        __syncthreads();
    }
    const uint32_t T = prefix;

    // 2. candidates: every token with key >= T
    if (tid == 0) {
        s_n = 0;
        s_overflow = 0;
    }
    __syncthreads();
    for (int i = tid; i < V; i += TPB) {
        const float v = a.logits[i];
        if (order_key(v) >= T) {
            const int p = atomicAdd(&s_n, 1);
            if (p < CAP - SAMPLER_HMAX) {       // room left for every history token
                cv[p] = v;
                ci[p] = i;
            } else {
                s_overflow = 1;
            }
        }
    }
    __syncthreads();
    if (s_overflow) {
        // more ties at T than the list holds: keep the keys above T and the
        // lowest ids equal to T, need in all (one thread; only for
        // degenerate rows such as many equal logits)
        if (tid == 0) {
            int n = 0;
            for (int i = 0; i < V && n < CAP; ++i)
                if (order_key(a.logits[i]) > T) {
                    cv[n] = a.logits[i];
                    ci[n++] = i;
                }
            for (int i = 0; i < V && n < CAP && n < need; ++i)
                if (order_key(a.logits[i]) == T) {
                    cv[n] = a.logits[i];
                    ci[n++] = i;
                }
            s_n = n;
        }
        __syncthreads();
    }
    // 3. penalties of the distinct history tokens (first occurrence does it);
    // every thread reads the list length before any history token is added
    const int n_base = min(s_n, CAP);
    __syncthreads();
    if (tid < a.n_hist) {
        const int t = a.hist[tid];
        bool first = true;
        int cnt = 0;
        for (int j = 0; j < a.n_hist; ++j) {
            const int tj = a.hist[j];
            cnt += tj == t;
            if (j < tid && tj == t) first = false;
        }
        if (first && t >= 0 && t < V) {
            float v = a.logits[t];
            v = v > 0.f ? v / a.pen_repeat : v * a.pen_repeat;
            v = v - (float)cnt * a.pen_freq - a.pen_present;
            int at = -1;
            for (int j = 0; j < n_base; ++j)
                if (ci[j] == t) at = j;
            if (at >= 0) {
                cv[at] = v;
            } else {
                const int p = atomicAdd(&s_n, 1);
                if (p < CAP) {
                    cv[p] = v;
                    ci[p] = t;
                }
            }
        }
    }
    __syncthreads();
    const int nc = min(s_n, CAP);
    // 4. bitonic sort of the next power of two >= nc slots (padding sorts last)
    int np2 = 2;
    while (np2 < nc) np2 <<= 1;
    for (int j = nc + tid; j < np2; j += TPB) {
        cv[j] = -INFINITY;
        ci[j] = 0x7FFFFFFF;
    }
    __syncthreads();
    for (int size = 2; size <= np2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int e = tid; e < np2 / 2; e += TPB) {
                const int lo = 2 * e - (e & (stride - 1));
                const int hi = lo + stride;
                const bool desc = (lo & size) == 0;      // this run sorts in "before" order
                const bool swap = desc ? before(cv[hi], ci[hi], cv[lo], ci[lo])
                                       : before(cv[lo], ci[lo], cv[hi], ci[hi]);
                if (swap) {
                    const float tv = cv[lo];
                    cv[lo] = cv[hi];
                    cv[hi] = tv;
                    const int ti = ci[lo];
                    ci[lo] = ci[hi];
                    ci[hi] = ti;
                }
            }
            __syncthreads();
        }
    }
    int n = min(a.top_k, nc);

    // 5. cut-offs on softmax weights (temperature 1), in the chain's order
    const float m = cv[0];
    if (a.top_p < 1.0f) {
        for (int j = tid; j < n; j += TPB) w[j] = expf(cv[j] - m);
        __syncthreads();
        block_scan(w, n);
        const float thr = a.top_p * w[n - 1];
        if (tid == 0) s_cut = n;
        __syncthreads();
        for (int j = tid; j < n; j += TPB)
            if (w[j] >= thr && (j == 0 || w[j - 1] < thr)) s_cut = j + 1;
        __syncthreads();
        n = s_cut;
        __syncthreads();
    }
    if (a.min_p > 0.0f) {
        // weights are non-increasing: keep the prefix with exp(v - m) >= min_p
        if (tid == 0) s_cut = n;
        __syncthreads();
        for (int j = tid; j < n; j += TPB) {
            const bool keep = expf(cv[j] - m) >= a.min_p;
            const bool keep_prev = j == 0 || expf(cv[j - 1] - m) >= a.min_p;
            if (!keep && keep_prev) s_cut = j;
        }
        __syncthreads();
        n = max(1, s_cut);
        __syncthreads();
    }
    // temperature and the draw
    int chosen = 0;
    if (a.temperature > 0.f) {
        for (int j = tid; j < n; j += TPB) w[j] = expf((cv[j] - m) / a.temperature);
        __syncthreads();
        block_scan(w, n);
        const float total = w[n - 1], thr = a.u * total;
        if (tid == 0) s_cut = n - 1;
        __syncthreads();
        for (int j = tid; j < n; j += TPB)
            if (w[j] > thr && (j == 0 || w[j - 1] <= thr)) s_cut = j;
        __syncthreads();
        chosen = s_cut;
        for (int j = tid; j < n && j < SAMPLER_KMAX; j += TPB) {
            a.out_ids[j] = ci[j];
            a.out_probs[j] = expf((cv[j] - m) / a.temperature) / total;
        }
    } else {
        for (int j = tid; j < n && j < SAMPLER_KMAX; j += TPB) {
            a.out_ids[j] = ci[j];
            a.out_probs[j] = j == 0 ? 1.f : 0.f;
        }
    }
    if (tid == 0) {
        a.out_token[0] = ci[chosen];
        a.out_token[1] = n;
    }
}

}  // namespace

void launch_sampler(const SamplerArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(sampler_kernel, dim3(1), dim3(TPB), 0, s, a);
}

}  // namespace ubd
