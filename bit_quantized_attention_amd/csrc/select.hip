// select.hip — ThriftAttention block selection for gfx950.
//
// "ThriftAttention" technical summary, Methodology step 1: the importance of
// the (query block i, key block j) pair is the dot product of the two blocks'
// mean vectors; per query block the top-k pairs over the causally valid key
// blocks run in 16-bit, with k = max(1, ceil(budget * n_valid)) (5 % in the
// Results).  Equal scores rank the smaller j first; the chosen j are written
// in ascending order.
//
// The scores decide integers (which blocks are chosen), so they are formed
// in fp64 exactly as the plain definition reads: products of the fp32 means
// (exact in fp64) summed channel by channel in ascending order, without
// fused multiply-add.  One workgroup per (b, query head, query block): the
// scores of all valid key blocks go to LDS, a bitonic sort orders them by
// (score descending, j ascending), and a second sort puts the first k block
// indices in ascending order.
#include <climits>

#include "common.hpp"
#include "internal.hpp"

#pragma clang fp contract(off)

namespace bqa {

namespace {

constexpr int NT = 256;

// a before b: higher score first, equal scores by smaller index
__device__ __forceinline__ bool before(double sa, int ja, double sb, int jb) {
    return sa > sb || (sa == sb && ja < jb);
}

__global__ __launch_bounds__(NT) void select_kernel(const float* __restrict__ qbar, const float* __restrict__ kbar,
                                                    int Hq, int Hkv, int nqb, int nkb, int d, int causal,
                                                    int budget_ppm, int max_sel, int L,
                                                    int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_cnt) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    double* sc = (double*)smem;                       // [L]
    int* jj = (int*)(smem + sizeof(double) * L);      // [L]
    __shared__ float q[128];

    const int tid = threadIdx.x;
    // The G = Hq / Hkv query heads of a KV head read the same key means: when
    // the (b, KV head) groups come in multiples of the 8 XCDs, workgroup id
    // 32-aligned blocks are arranged so that the G heads of a group share an
    // XCD (ids that differ by multiples of 8), and its L2.
    const int G = Hq / Hkv, nbk = (int)(gridDim.x / nqb) / G;   // (b, KV head) groups
    int bh, i;
    if (nbk % 8 == 0) {
        const int id = blockIdx.x, x = id % 8, rest = id / 8;   // XCD, then (group block, head, query block)
        i = rest % nqb;
        const int hh = (rest / nqb) % G, a = rest / nqb / G;
        const int grp = 8 * a + x;                              // b * Hkv + KV head
        bh = (grp / Hkv) * Hq + (grp % Hkv) * G + hh;
    } else {
        i = blockIdx.x % nqb;
        bh = blockIdx.x / nqb;
    }
    const int b = bh / Hq, h = bh % Hq;                 // bh = b * Hq + h
    const int hk = h / G;
    const float* qrow = qbar + ((int64_t)bh * nqb + i) * d;
    const float* kb = kbar + ((int64_t)b * Hkv + hk) * nkb * d;
    for (int c = tid; c < d; c += NT) q[c] = qrow[c];
    __syncthreads();

    int nv = causal ? i + (nkb - nqb) + 1 : nkb;
    if (nv > nkb) nv = nkb;
    if (nv < 0) nv = 0;
    for (int j = tid; j < L; j += NT) {
        double acc = -__builtin_inf();
        int jv = INT_MAX;
        if (j < nv) {
            const float* kr = kb + (int64_t)j * d;
            acc = 0.0;
            for (int c = 0; c < d; c += 4) {
                const float4 k4 = *(const float4*)(kr + c);
                acc = acc + (double)q[c + 0] * (double)k4.x;
                acc = acc + (double)q[c + 1] * (double)k4.y;
                acc = acc + (double)q[c + 2] * (double)k4.z;
                acc = acc + (double)q[c + 3] * (double)k4.w;
            }
            jv = j;
        }
        sc[j] = acc;
        jj[j] = jv;
    }
    __syncthreads();

    // bitonic sort of L (power of two) entries into "before" order
    for (int k = 2; k <= L; k <<= 1) {
        for (int s = k >> 1; s > 0; s >>= 1) {
            for (int t = tid; t < L / 2; t += NT) {
                const int a = 2 * s * (t / s) + (t % s), c = a + s;
                const bool up = (a & k) == 0;
                const double sa = sc[a], sb = sc[c];
                const int ja = jj[a], jb = jj[c];
                if (before(sb, jb, sa, ja) == up) {
                    sc[a] = sb; sc[c] = sa;
                    jj[a] = jb; jj[c] = ja;
                }
            }
            __syncthreads();
        }
    }

    // k = max(1, ceil(n_valid * budget)), at most n_valid and max_sel
    int kk = 0;
    if (nv > 0) {
        const int64_t want = ((int64_t)nv * budget_ppm + 999999) / 1000000;
        kk = (int)(want < 1 ? 1 : (want > nv ? nv : want));
        if (kk > max_sel) kk = max_sel;
    }
    int P = 1;
    while (P < kk) P <<= 1;
    // the chosen indices, ascending: reuse the first P slots of jj as keys
    __syncthreads();
    for (int t = tid; t < P; t += NT) {
        if (t >= kk) jj[t] = INT_MAX;
    }
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1) {
        for (int s = k >> 1; s > 0; s >>= 1) {
            for (int t = tid; t < P / 2; t += NT) {
                const int a = 2 * s * (t / s) + (t % s), c = a + s;
                const bool up = (a & k) == 0;
                const int ja = jj[a], jb = jj[c];
                if ((ja > jb) == up) { jj[a] = jb; jj[c] = ja; }
            }
            __syncthreads();
        }
    }
    int32_t* out = sel_idx + ((int64_t)bh * nqb + i) * max_sel;
    for (int t = tid; t < max_sel; t += NT) out[t] = t < kk ? jj[t] : -1;
    if (tid == 0) sel_cnt[(int64_t)bh * nqb + i] = kk;
}

}  // namespace

int select_sort_len(int nkb) {
    int L = 1;
    while (L < nkb) L <<= 1;
    return L < 2 ? 2 : L;
}

hipError_t launch_select(const float* qbar, const float* kbar, int B, int Hq, int Hkv, int nqb, int nkb, int d,
                         int causal, int budget_ppm, int max_sel, int32_t* sel_idx, int32_t* sel_cnt,
                         hipStream_t st) {
    const int L = select_sort_len(nkb);
    const size_t shm = (size_t)L * (sizeof(double) + sizeof(int));
    select_kernel<<<B * Hq * nqb, NT, shm, st>>>(qbar, kbar, Hq, Hkv, nqb, nkb, d, causal, budget_ppm, max_sel, L,
                                                 sel_idx, sel_cnt);
    return hipGetLastError();
}

}  // namespace bqa
