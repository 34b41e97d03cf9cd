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
// scores of all valid key blocks go to LDS, and a radix selection on their
// order-preserving 64-bit keys (eight bits per pass) finds the k-th largest; the blocks above it,
// and of those equal to it the ones with the smallest j, are written in
// ascending order through prefix counts.  Nothing is sorted.
#include <climits>

#include "common.hpp"
#include "internal.hpp"

#pragma clang fp contract(off)

namespace bqa {

namespace {

constexpr int NT = 256;

// Exclusive prefix sum over the workgroup of one count per thread (thread
// order), and the total.  Holds workgroup barriers; `ws` is NT / 64 ints of
// LDS used only inside.
__device__ __forceinline__ int block_excl_scan(int v, int tid, int* ws, int& total) {
    const int l = tid & 63;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __builtin_amdgcn_ds_bpermute(4 * (l >= o ? l - o : l), incl);
        if (l >= o) incl += u;
    }
    __syncthreads();                                  // ws is free
    if (l == 63) ws[tid >> 6] = incl;
    __syncthreads();
    int pre = incl - v;
    total = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const int x = ws[w];
        if (w < (tid >> 6)) pre += x;
        total += x;
    }
    return pre;
}

// Order-preserving 64-bit key of a score: larger score, larger key.
__device__ __forceinline__ uint64_t score_key(double s) {
    const uint64_t b = (uint64_t)__double_as_longlong(s);
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// Top kk of the L <= 4096 scores sc[0..L) (block j's score at j; entries
// without a block are -inf) in "before" order, written as block indices in
// ascending order to out[0..kk), out[kk..max_sel) = -1.  Radix selection on
// the order-preserving keys, eight bits per pass from the top: each pass
// histograms the next digit of the keys that share the prefix so far (one
// LDS histogram per wavefront, atomic adds) and keeps the digit where the
// kk-th largest key falls.  The chosen blocks are those above the resulting
// threshold key and, of those equal to it, the ones with the smallest
// indices (equal scores rank the smaller j first).  Thread t owns entries
// E t .. E t + E - 1 (E = L / NT, at least 1).  `hist` is 2 x 4 x 256 ints of
// LDS.  Holds workgroup barriers.
__device__ __forceinline__ void radix_topk(const double* sc, int L, int kk, int32_t* out, int max_sel, int tid,
                                           int* hist) {
    __shared__ int ws[NT / 64];
    __shared__ int pick[2][2];                        // per pass parity: digit, keys above it
    const int E = L >= NT ? L / NT : 1, w = tid >> 6, l = tid & 63;
    uint64_t key[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const int e = E * tid + u;
        key[u] = (u < E && e < L) ? score_key(sc[e]) : 0ull;     // 0: below every score's key
    }
    for (int x = tid; x < 2 * 4 * 256; x += NT) hist[x] = 0;
    __syncthreads();
    uint64_t pre = 0;                                 // threshold bits decided so far
    int need = kk;                                    // rank of the threshold among keys with that prefix
    if (kk > 0) {
        for (int pass = 0; pass < 8; ++pass) {
            const int sh = 56 - 8 * pass;
            int* hb = hist + (pass & 1) * 1024;
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                if (u < E && (pass == 0 || (key[u] >> (sh + 8)) == pre))
                    atomicAdd(hb + 256 * w + (int)((key[u] >> sh) & 255u), 1);
            }
            __syncthreads();
            if (w == 0) {
                // lane l sums bins 255 - 4 l .. 252 - 4 l over the wavefronts (top bins first)
                int c4[4], s4 = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int bin = 255 - 4 * l - q;
                    c4[q] = hb[bin] + hb[256 + bin] + hb[512 + bin] + hb[768 + bin];
                    s4 += c4[q];
                }
                int incl = s4;                        // keys in the bins above and at this lane's four
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const int v = __builtin_amdgcn_ds_bpermute(4 * (l >= o ? l - o : l), incl);
                    if (l >= o) incl += v;
                }
                int above = incl - s4;
                if (above < need && need <= incl) {   // exactly one lane
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if (above + c4[q] >= need) { pick[pass & 1][0] = 255 - 4 * l - q; pick[pass & 1][1] = above; break; }
                        above += c4[q];
                    }
                }
            }
            // the other parity's histogram is cleared for the pass after next
            int* hc = hist + ((pass + 1) & 1) * 1024;
            for (int x = tid; x < 1024; x += NT) hc[x] = 0;
            __syncthreads();
            const int dig = pick[pass & 1][0];
            need -= pick[pass & 1][1];
            pre = (pre << 8) | (uint64_t)dig;
        }
    }
    // chosen: key > pre, or key == pre among the first `need` such blocks (ascending j)
    int n_eq = 0;
#pragma unroll
    for (int u = 0; u < 16; ++u)
        if (u < E && kk > 0 && key[u] == pre) ++n_eq;
    int tot;
    int eq_rank = block_excl_scan(n_eq, tid, ws, tot);
    int n_sel = 0;
    bool sel[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        bool c = false;
        if (u < E && kk > 0) {
            if (key[u] > pre) c = true;
            else if (key[u] == pre) c = eq_rank++ < need;
        }
        sel[u] = c;
        n_sel += c;
    }
    int pos = block_excl_scan(n_sel, tid, ws, tot);
#pragma unroll
    for (int u = 0; u < 16; ++u)
        if (sel[u]) out[pos++] = E * tid + u;
    for (int t = kk + tid; t < max_sel; t += NT) out[t] = -1;
}

__global__ __launch_bounds__(NT) void select_kernel(const float* __restrict__ qbar, const float* __restrict__ kbar,
                                                    int Hq, int Hkv, int nqb, int nkb, int d, int causal,
                                                    int budget_ppm, int max_sel, int L, int ring,
                                                    int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_cnt) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    double* sc = (double*)smem;                       // [L]: block j's score at j
    uint8_t* kt = smem + sizeof(double) * L;          // ring: 3 x [NT][64 B] pieces of the key means; then 8 KB of histograms
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
    // Scores of the valid key blocks, thread t owning block r0 + t of each
    // chunk of NT blocks.  The key means pass through LDS in pieces of 16
    // channels x NT blocks (16 KB), in a ring of three slots, by direct
    // global -> LDS copies: each wavefront copies four 1 KB segments of a
    // piece, lane l landing at segment base + 16 l; the source each lane
    // names puts chunk c (4 channels) of block row t at 16-byte slot
    // c ^ ((t >> 2) & 3) of the row's 64 bytes, so that 16 consecutive
    // threads reading the same chunk of their own rows hit 16 different
    // bank groups.  Two pieces are in flight while one is summed; the
    // running sum carries over the pieces of a chunk, so the channels are
    // still added in ascending order.
    for (int j = tid; j < L; j += NT) sc[j] = -__builtin_inf();
    if (!ring) {
        // many workgroups (prefill) or long rows: each thread reads its rows
        // directly, and the small LDS footprint lets 8 workgroups share a CU
        for (int j = tid; j < nv; j += NT) {
            const float* kr = kb + (int64_t)j * d;
            double a = 0.0;
            for (int c = 0; c < d; c += 4) {
                const float4 k4 = *(const float4*)(kr + c);
                a = a + (double)q[c + 0] * (double)k4.x;
                a = a + (double)q[c + 1] * (double)k4.y;
                a = a + (double)q[c + 2] * (double)k4.z;
                a = a + (double)q[c + 3] * (double)k4.w;
            }
            sc[j] = a;
        }
    }
    const int npc = d / 16, nch = ring ? (nv + NT - 1) / NT : 0, n_pieces = nch * npc;
    const int wv = tid >> 6, ln = tid & 63;
    auto issue = [&](int pc) __attribute__((always_inline)) {
        const int r0 = pc / npc * NT, c0 = pc % npc * 16;
        uint8_t* slot = kt + (pc % 3) * (NT * 64);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int sg = 4 * wv + u, t = 16 * sg + (ln >> 2), c = (ln & 3) ^ ((t >> 2) & 3);
            const int row = r0 + t < nv ? r0 + t : nv - 1;            // rows past nv are never summed
            lds_copy16((uint32_t)((row * d + c0 + 4 * c) * 4), kb, lds_addr(slot + 1024 * sg));
        }
    };
    if (n_pieces > 0) issue(0);
    if (n_pieces > 1) issue(1);
    double acc = 0.0;
    for (int pc = 0; pc < n_pieces; ++pc) {
        if (pc + 1 < n_pieces) BQA_WAIT_VM(4);                        // this wavefront's copies of piece pc
        else BQA_WAIT_VM(0);
        barrier_only();                                               // everyone's copies of pc; pc - 1 is read
        if (pc + 2 < n_pieces) issue(pc + 2);
        const int r0 = pc / npc * NT, c0 = pc % npc * 16;
        if (c0 == 0) acc = 0.0;
        const uint8_t* row = kt + (pc % 3) * (NT * 64) + 64 * tid;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float4 k4 = *(const float4*)(row + 16 * (c ^ ((tid >> 2) & 3)));
            acc = acc + (double)q[c0 + 4 * c + 0] * (double)k4.x;
            acc = acc + (double)q[c0 + 4 * c + 1] * (double)k4.y;
            acc = acc + (double)q[c0 + 4 * c + 2] * (double)k4.z;
            acc = acc + (double)q[c0 + 4 * c + 3] * (double)k4.w;
        }
        if (c0 + 16 == d && r0 + tid < nv) sc[r0 + tid] = acc;
    }
    __syncthreads();

    // k = max(1, ceil(n_valid * budget)), at most n_valid and max_sel
    int kk = 0;
    if (nv > 0) {
        const int64_t want = ((int64_t)nv * budget_ppm + 999999) / 1000000;
        kk = (int)(want < 1 ? 1 : (want > nv ? nv : want));
        if (kk > max_sel) kk = max_sel;
    }
    int32_t* out = sel_idx + ((int64_t)bh * nqb + i) * max_sel;
    if (tid == 0) sel_cnt[(int64_t)bh * nqb + i] = kk;

    radix_topk(sc, L, kk, out, max_sel, tid, (int*)kt);             // the histograms reuse the pieces' LDS
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
    const size_t shm = (size_t)L * sizeof(double);
    // The LDS ring of key-mean pieces serves rows of up to 1024 blocks when
    // the grid is small enough that the time of one workgroup is the time of
    // the launch (decode: 512 workgroups); a large grid (prefill, one
    // workgroup per query block) is throughput-bound and takes the direct
    // row reads with a small LDS footprint.
    const int grid = B * Hq * nqb;
    const int ring = L <= 1024 && grid <= 4096;
    const size_t lds = shm + (ring ? 3 * NT * 64 : 8192);     // at most 56 KB
    select_kernel<<<grid, NT, lds, st>>>(qbar, kbar, Hq, Hkv, nqb, nkb, d, causal, budget_ppm, max_sel, L, ring,
                                         sel_idx, sel_cnt);
    return hipGetLastError();
}

}  // namespace bqa
