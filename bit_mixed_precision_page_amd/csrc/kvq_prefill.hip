// kvq_prefill.hip -- prefill attention of one sequence with cumulative
// attention scores, and heavy-hitter + recent token selection (gfx950).
//
// MiniKV summary (f-binder), "proposed method": the prefill processes the
// whole input and chooses the KV states to keep from cumulative attention
// scores -- the heavy hitters plus a recent window, 25 % of the budget each by
// default -- and a two-stage selective flash-attention yields the attention
// output and the cumulative scores in linear memory.  Readings: the attention
// is causal; the score of key position j is the sum, over the query heads of
// its KV head and the query rows i >= j, of the softmax probability P[i][j];
// the last `recent` positions are kept, plus the `heavy` positions of largest
// score among the others (ties to the lower position), listed ascending.
//
// Stage 0  Values transposed per 32-key block to [Hkv][T32 / 32][D][32]
//          (T32 = T rounded up to 32, zero tail), keys in the order a lane of
//          the transposed score tile holds them: a lane's P.V operand is one
//          16-byte read.
// Stage 1  flash attention: four-wave workgroups over the query heads of
//          one KV head (up to four) and 32 query rows per wave; each 32-key
//          block of Keys and Values is staged once in LDS for the workgroup
//          (double buffered).  S^T = K Q^T on the matrix cores (the dtype
//          inputs are exact, fp32 accumulation); online softmax in the log2
//          domain; P^T split into a dtype hi and lo part (~16 bits for bf16,
//          ~22 for fp16) feeds O^T = V^T P^T directly, 2 MFMAs per
//          16-channel tile.  Writes out (fp32) and per row the log2 of the
//          softmax denominator.  A short sequence (too few workgroups for
//          the chip) splits each row block's keys into chunks whose
//          unnormalized partials a merge kernel combines.
// Stage 2  cumulative scores: four-wave workgroups over 256 keys of one KV
//          head and a chunk of query rows, Key operands in registers, the
//          query blocks of every query head of the group streamed through
//          LDS: S again, P = 2^(s qscale - lse_i) with the row's log2
//          softmax denominator from stage 1, column sums in registers; a second kernel adds the
//          chunks' partial sums in chunk order, so the scores do not depend
//          on scheduling.
// Stage 3  selection, one workgroup per KV head: the heavy-th largest score
//          by a radix select over the score bits, 8 bits per pass (scores
//          are >= 0, so the bits order like the values), ties at that score
//          resolved to the lower positions by a prefix count, then an
//          ascending compaction.
// Stage 4  gather of the kept K and V rows.
#include "kvq_decode_core.h"

namespace kvq {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelCache = 16384;  // scores cached in LDS (64 KB)

// fp32 pair -> dtype pair, round to nearest even
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    if constexpr (DT == F16) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{a, b}, h2_t));
    } else {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{a, b}, bf2_t));
    }
}
template <int DT>
__device__ __forceinline__ float lo16(uint32_t w) {
    return dec<DT>((uint16_t)(w & 0xffffu));
}
template <int DT>
__device__ __forceinline__ float hi16(uint32_t w) {
    return dec<DT>((uint16_t)(w >> 16));
}

// max / sum over the four lanes r, r + 16, r + 32, r + 48 (the four rows of
// the wave), in all four: v_permlane32_swap of a register with itself pairs
// rows 0, 1 with rows 2, 3; v_permlane16_swap pairs even rows with odd rows.
__device__ __forceinline__ float xrow_max(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xrow_sum(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Key of slot s in a 32-key block of the Value operand: slots 8 b + [0, 4)
// hold keys 4 b + [0, 4) and slots 8 b + [4, 8) keys 16 + 4 b + [0, 4), the
// keys a lane of the transposed score tiles holds (see prefill_fwd_kernel).
__device__ __forceinline__ int slot_key(int s) {
    const int b = s >> 3, e = s & 7;
    return e < 4 ? 4 * b + e : 12 + 4 * b + e;
}

// ---------------------------------------------------------------- stage 0
// vt[h][blk][c][s] = v[h][32 blk + slot_key(s)][c], zero past T: each
// 32-key block's transposed Values are one contiguous 8 KB.
__global__ __launch_bounds__(256) void v_transpose_kernel(const uint16_t *__restrict__ v,
                                                          uint16_t *__restrict__ vt, int T,
                                                          int T32) {
    __shared__ uint16_t tile[32][D + 8];
    const int h = blockIdx.y, blk = blockIdx.x, t0 = blk * 32, tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; i++) {  // 32 tokens x 16 chunks of 8 channels
        const int x = tid + 256 * i, tok = x >> 4, c8 = x & 15;
        uint4 w = make_uint4(0, 0, 0, 0);
        if (t0 + tok < T) w = *reinterpret_cast<const uint4 *>(v + ((size_t)h * T + t0 + tok) * D + 8 * c8);
        *reinterpret_cast<uint4 *>(&tile[tok][8 * c8]) = w;
    }
    __syncthreads();
    const int c = tid >> 1, half = tid & 1;  // channel c, slots 16 half + [0, 16)
    uint32_t o[8];
#pragma unroll
    for (int e = 0; e < 8; e++) {
        const int s = 16 * half + 2 * e;
        o[e] = (uint32_t)tile[slot_key(s)][c] | ((uint32_t)tile[slot_key(s + 1)][c] << 16);
    }
    uint4 *dst = reinterpret_cast<uint4 *>(vt + (((size_t)h * (T32 / 32) + blk) * D + c) * 32 + 16 * half);
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

// ---------------------------------------------------------------- stage 1
// Workgroup of four waves = hw query heads of one KV head x 4 / hw groups of
// 32 query rows (hw = 4, 2 or 1, dividing the group size); a wave owns 32
// rows (two 16-row tiles) of one query head.  Each 32-key block of Keys and
// transposed Values (16 KB) is loaded once per workgroup into LDS (double
// buffered, the next block's global loads in flight during this block's
// math) and read by every wave; each operand read serves both row tiles.
// The scores are computed transposed, S^T = K Q^T: a lane then holds one
// query row and keys 4 b + e, 16 + 4 b + e of the block, which is directly
// the B operand of O^T = V^T P^T once the Values are stored in the slot
// order of slot_key -- no transpose of P.
constexpr int kKRow = D + 8;          // LDS Key row (272 B: consecutive rows start 4 banks apart)
constexpr int kVRow = 40;             // LDS Value row, 32 slots + pad (80 B: 20 banks apart)
constexpr int kKTile = 32 * kKRow;    // elements
constexpr int kFwdBuf = kKTile + D * kVRow;

// Online softmax of one 32-key block for the wave's two row tiles.  The
// reference maximum of a row moves only when a block's maximum exceeds it by
// more than kRescaleSlack (log2 units), so P stays below 2^kRescaleSlack and
// the accumulators are rescaled only in the first blocks of a row.  P^T goes
// out as a dtype hi and lo part, the B operands of O^T = V^T P^T.
constexpr float kRescaleSlack = 8.0f;
template <int DT, bool MASK>
__device__ __forceinline__ void block_softmax(const f4_t (&s)[2][2], int j0, int i0w, int T,
                                              float qscale, float (&m_run)[2], float (&l_run)[2],
                                              float (&alpha)[2], bool (&up)[2], u4_t (&bhi)[2],
                                              u4_t (&blo)[2], int r, int kb) {
#pragma unroll
    for (int u = 0; u < 2; u++) {
        float x[8];
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                if constexpr (MASK) {
                    const int i = min(i0w + 16 * u + r, T - 1), j = j0 + 16 * t + 4 * kb + e;
                    x[4 * t + e] = j <= i ? s[u][t][e] : -INFINITY;
                } else {
                    x[4 * t + e] = s[u][t][e];
                }
            }
        float bm = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                         fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        // every visited block holds a key <= the row, so the block maximum is finite
        bm = xrow_max(bm) * qscale;
        const bool grow = bm > m_run[u] + kRescaleSlack;
        const float mn = grow ? bm : m_run[u];
        alpha[u] = __builtin_amdgcn_exp2f(m_run[u] - mn);
        up[u] = __any(grow);  // wave-uniform
        m_run[u] = mn;
        float ps = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            x[e] = __builtin_amdgcn_exp2f(fmaf(x[e], qscale, -mn));
            ps += x[e];
        }
        l_run[u] = fmaf(l_run[u], alpha[u], ps);
#pragma unroll
        for (int d = 0; d < 4; d++) {
            const uint32_t hw2 = pack2<DT>(x[2 * d], x[2 * d + 1]);
            bhi[u][d] = hw2;
            blo[u][d] = pack2<DT>(x[2 * d] - lo16<DT>(hw2), x[2 * d + 1] - hi16<DT>(hw2));
        }
    }
}

template <int DT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void prefill_fwd_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ vt, float *__restrict__ out, float *__restrict__ lse, int T,
    int T32, int g, int hw, float qscale, int kbc, int nsplit, float *__restrict__ pml,
    float *__restrict__ pacc) {
    __shared__ __align__(16) uint16_t lds[2 * kFwdBuf];
    const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, kb = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hq = blockIdx.x * hw + w % hw, h = blockIdx.x * hw / g;
    const int qr = 128 / hw;  // query rows of the workgroup
    // the last query rows see the most keys: dispatched first
    const int i0g = (gridDim.y - 1 - blockIdx.y) * qr;
    const int i0w = i0g + 32 * (w / hw);
    const int nbg = (min(T - 1, i0g + qr - 1)) / 32 + 1;
    const int nbw = i0w < T ? (min(T - 1, i0w + 31)) / 32 + 1 : 0;
    const int nb = T32 / 32;
    const uint16_t *kh = k + (size_t)h * T * D;
    const uint16_t *vth = vt + (size_t)h * nb * D * 32;
    // key chunk of this workgroup: blocks [jb0, jb1) (every block when the
    // keys are not split)
    const int chunk = blockIdx.z, jb0 = chunk * kbc;
    if (jb0 >= nbg) return;  // workgroup-uniform: no key of the chunk precedes its rows
    const int jb1 = min(nbg, jb0 + kbc);

    // block jb -> registers (two 16-byte pieces of Keys and two of Values per thread)
    u4_t pk[2], pv[2];
    auto gload = [&](int jb) {
        const int j0 = 32 * jb;
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int c = tid + 256 * i, key = c >> 4, c8 = c & 15;
            pk[i] = j0 + key < T ? *reinterpret_cast<const u4_t *>(kh + (size_t)(j0 + key) * D + 8 * c8)
                                 : u4_t{0, 0, 0, 0};
            pv[i] = *reinterpret_cast<const u4_t *>(vth + (size_t)jb * D * 32 + 8 * c);
        }
    };
    auto lstore = [&](int buf) {
        uint16_t *L = lds + buf * kFwdBuf;
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int c = tid + 256 * i;
            *reinterpret_cast<u4_t *>(L + (c >> 4) * kKRow + 8 * (c & 15)) = pk[i];
            *reinterpret_cast<u4_t *>(L + kKTile + (c >> 2) * kVRow + 8 * (c & 3)) = pv[i];
        }
    };

    // B operand of S^T: query row i0w + 16 u + r, channels 32 m + 8 kb + [0, 8)
    u4_t aq[2][4];
#pragma unroll
    for (int u = 0; u < 2; u++) {
        const uint16_t *qrow = q + ((size_t)hq * T + min(i0w + 16 * u + r, T - 1)) * D;
#pragma unroll
        for (int m = 0; m < 4; m++) aq[u][m] = *reinterpret_cast<const u4_t *>(qrow + 32 * m + 8 * kb);
    }
    float m_run[2], l_run[2];  // reference row max (log2 units); this lane's part of the row sum
    f4_t acc[2][8];            // O^T: row i0w + 16 u + r, channels 16 n + 4 kb + e
#pragma unroll
    for (int u = 0; u < 2; u++) {
        m_run[u] = -INFINITY;
        l_run[u] = 0.0f;
#pragma unroll
        for (int n = 0; n < 8; n++) acc[u][n] = f4_t{0, 0, 0, 0};
    }

    gload(jb0);
    lstore(jb0 & 1);
    if (jb0 + 1 < jb1) gload(jb0 + 1);
    for (int jb = jb0; jb < jb1; jb++) {
        __syncthreads();  // block jb is in LDS; every wave is done with block jb - 1
        if (jb + 1 < jb1) lstore((jb + 1) & 1);
        if (jb + 2 < jb1) gload(jb + 2);
        if (jb >= nbw) continue;
        const uint16_t *L = lds + (jb & 1) * kFwdBuf;
        const int j0 = 32 * jb;
        f4_t s[2][2];
#pragma unroll
        for (int t = 0; t < 2; t++) {
            s[0][t] = f4_t{0, 0, 0, 0};
            s[1][t] = f4_t{0, 0, 0, 0};
#pragma unroll
            for (int m = 0; m < 4; m++) {
                const u4_t ka = *reinterpret_cast<const u4_t *>(L + (16 * t + r) * kKRow + 32 * m + 8 * kb);
                s[0][t] = mfma_dt<DT>(ka, aq[0][m], s[0][t]);
                s[1][t] = mfma_dt<DT>(ka, aq[1][m], s[1][t]);
            }
        }
        u4_t bhi[2], blo[2];
        // the mask matters only where keys pass the wave's first row (the
        // diagonal block, which also holds any keys past T)
        float alpha[2];
        bool up[2];
        if (j0 + 31 > i0w)
            block_softmax<DT, true>(s, j0, i0w, T, qscale, m_run, l_run, alpha, up, bhi, blo, r, kb);
        else
            block_softmax<DT, false>(s, j0, i0w, T, qscale, m_run, l_run, alpha, up, bhi, blo, r, kb);
#pragma unroll
        for (int u = 0; u < 2; u++)
            if (up[u]) {
#pragma unroll
                for (int n = 0; n < 8; n++) acc[u][n] *= alpha[u];
            }
        // the P.V products at a raised issue priority (s_setprio) against the
        // other waves of the SIMD: 2 % less time for this kernel, measured
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int n = 0; n < 8; n++) {
            const u4_t va = *reinterpret_cast<const u4_t *>(L + kKTile + (16 * n + r) * kVRow + 8 * kb);
#pragma unroll
            for (int u = 0; u < 2; u++) {
                acc[u][n] = mfma_dt<DT>(va, bhi[u], acc[u][n]);
                acc[u][n] = mfma_dt<DT>(va, blo[u], acc[u][n]);
            }
        }
        __builtin_amdgcn_s_setprio(0);
    }
    if (nsplit > 1) {
        // unnormalized partials of this key chunk; a wave whose rows end
        // before the chunk writes none (the merge does not read them)
        if (jb0 >= nbw) return;
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const float l = xrow_sum(l_run[u]);
            const int i = i0w + 16 * u + r;
            if (i < T) {
                const size_t pr = ((size_t)hq * T + i) * nsplit + chunk;
                float *o = pacc + pr * D + 4 * kb;
#pragma unroll
                for (int n = 0; n < 8; n++) *reinterpret_cast<f4_t *>(o + 16 * n) = acc[u][n];
                if (kb == 0) *reinterpret_cast<float2 *>(pml + 2 * pr) = make_float2(m_run[u], l);
            }
        }
        return;
    }
#pragma unroll
    for (int u = 0; u < 2; u++) {
        const float l = xrow_sum(l_run[u]);
        const int i = i0w + 16 * u + r;
        if (i < T) {
            const float inv = 1.0f / l;
            float *o = out + ((size_t)hq * T + i) * D + 4 * kb;
#pragma unroll
            for (int n = 0; n < 8; n++)
                *reinterpret_cast<f4_t *>(o + 16 * n) = acc[u][n] * inv;
            // log2 of the row's softmax denominator: P[i][j] = 2^(s_ij qscale - lse)
            if (kb == 0) lse[(size_t)hq * T + i] = m_run[u] + __builtin_amdgcn_logf(l);
        }
    }
}

// Key-split attention: row (hq, i) combines the partials of the chunks that
// hold keys <= i, one wave per row, two channels per lane.
__global__ __launch_bounds__(256) void prefill_merge_kernel(const float *__restrict__ pml,
                                                            const float *__restrict__ pacc,
                                                            float *__restrict__ out,
                                                            float *__restrict__ lse, int T,
                                                            int rows, int nsplit, int kbc) {
    const int row = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const int i = row % T, nch = min(nsplit, (i / 32) / kbc + 1);
    float2 st[kPrefillMaxKeySplits], x[kPrefillMaxKeySplits];
    float M = -INFINITY;
#pragma unroll
    for (int c = 0; c < kPrefillMaxKeySplits; c++) {
        if (c < nch) {
            const size_t pr = (size_t)row * nsplit + c;
            st[c] = *reinterpret_cast<const float2 *>(pml + 2 * pr);
            x[c] = *reinterpret_cast<const float2 *>(pacc + pr * D + 2 * lane);
            M = fmaxf(M, st[c].x);
        }
    }
    float L = 0.0f, ax = 0.0f, ay = 0.0f;
#pragma unroll
    for (int c = 0; c < kPrefillMaxKeySplits; c++) {
        if (c < nch) {
            const float w = __builtin_amdgcn_exp2f(st[c].x - M);
            L = fmaf(w, st[c].y, L);
            ax = fmaf(w, x[c].x, ax);
            ay = fmaf(w, x[c].y, ay);
        }
    }
    const float inv = 1.0f / L;
    *reinterpret_cast<float2 *>(out + (size_t)row * D + 2 * lane) = make_float2(ax * inv, ay * inv);
    if (lane == 0) lse[row] = M + __builtin_amdgcn_logf(L);
}

// ---------------------------------------------------------------- stage 2
// Workgroup (kCsKeys keys, query chunk, KV head) of four waves, kCsKT 16-key
// tiles per wave, the Key operands held in registers.  The
// workgroup streams the 32-row query blocks of its chunk at or after its
// keys, for every query head of the group, through LDS (double buffered,
// with the row statistics); each Q operand read serves the wave's kCsKT key
// tiles.  S = Q K^T puts one key per lane and four query rows per result
// register, so the column sums accumulate in registers.  The partial sums go
// to part[h][y][T] and a second kernel adds the chunks in order: the scores
// do not depend on scheduling.
constexpr int kCsKT = 4;                   // 16-key tiles per wave
constexpr int kCsKeys = 4 * 16 * kCsKT;    // keys per workgroup
constexpr int kCsRows = 64;                // query rows per step
constexpr int kCsBuf = kCsRows * kKRow;    // elements of one staged query block

// column sums of one 16-row tile against the wave's kCsKT key tiles
template <int DT, bool MASK>
__device__ __forceinline__ void tile_colsum(const u4_t (&aq)[4], const u4_t (&bk)[kCsKT][4],
                                            const float (&st)[4], float (&cs)[kCsKT], int i0,
                                            int jw, int T, float qscale, int r, int kb) {
#pragma unroll
    for (int kt = 0; kt < kCsKT; kt++) {
        f4_t c = {0, 0, 0, 0};
#pragma unroll
        for (int m = 0; m < 4; m++) c = mfma_dt<DT>(aq[m], bk[kt][m], c);
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const float pr = __builtin_amdgcn_exp2f(fmaf(c[e], qscale, -st[e]));
            if constexpr (MASK) {
                const int i = i0 + 4 * kb + e, j = jw + 16 * kt + r;
                cs[kt] += i < T && j <= i ? pr : 0.0f;
            } else {
                cs[kt] += pr;
            }
        }
    }
}

// key blocks of kCsKeys with a query row of chunk y at or after their first key
__host__ __device__ __forceinline__ int cs_blocks(int y, int cr, int T) {
    const int nkb = (T + kCsKeys - 1) / kCsKeys;
    return min(nkb, (min(T, (y + 1) * cr) + kCsKeys - 1) / kCsKeys);
}

template <int DT>
__global__ __launch_bounds__(256) void prefill_colsum_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const float *__restrict__ lse, float *__restrict__ part, int T, int g, float qscale, int cr,
    int nchunk) {
    __shared__ __align__(16) uint16_t lq[2 * kCsBuf];
    __shared__ float lst[2][kCsRows];
    const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, kb = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // only the (key block, chunk) pairs with a row at or after a key are
    // launched: chunk y holds cs_blocks(y) key blocks; the last chunks first
    const int h = blockIdx.y;
    int chunk = nchunk - 1, kx = blockIdx.x;
    while (kx >= cs_blocks(chunk, cr, T)) kx -= cs_blocks(chunk--, cr, T);
    const int jg = kCsKeys * kx, jw = jg + 16 * kCsKT * w;
    float *dst = part + ((size_t)h * nchunk + chunk) * T;
    // query rows [r0, r1): the chunk's rows from the first key (cr and the key
    // blocks are multiples of kCsRows, so steps never cross into another chunk)
    const int r0 = max(chunk * cr, jg), r1 = min(T, chunk * cr + cr);
    u4_t bk[kCsKT][4];  // B operand: key jw + 16 kt + r, channels 32 m + 8 kb + [0, 8)
#pragma unroll
    for (int kt = 0; kt < kCsKT; kt++) {
        const uint16_t *krow = k + ((size_t)h * T + min(jw + 16 * kt + r, T - 1)) * D;
#pragma unroll
        for (int m = 0; m < 4; m++) bk[kt][m] = *reinterpret_cast<const u4_t *>(krow + 32 * m + 8 * kb);
    }
    const int nsteps = g * ((r1 - r0 + kCsRows - 1) / kCsRows);
    // steps run over (query head h g + a, rows rb + [0, kCsRows)), rb from r0 to r1
    int la = 0, lrb = r0;  // the next step to load
    u4_t pq[kCsRows / 16];
    float ps;
    auto gload = [&]() {
        const int hq = h * g + la;
#pragma unroll
        for (int i = 0; i < kCsRows / 16; i++) {
            const int c = tid + 256 * i, row = c >> 4, c8 = c & 15;
            pq[i] = lrb + row < T ? *reinterpret_cast<const u4_t *>(q + ((size_t)hq * T + lrb + row) * D + 8 * c8)
                                  : u4_t{0, 0, 0, 0};
        }
        if (tid < kCsRows) ps = lrb + tid < T ? lse[(size_t)hq * T + lrb + tid] : 0.0f;
        lrb += kCsRows;
        if (lrb >= r1) {
            lrb = r0;
            la++;
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < kCsRows / 16; i++) {
            const int c = tid + 256 * i;
            *reinterpret_cast<u4_t *>(lq + buf * kCsBuf + (c >> 4) * kKRow + 8 * (c & 15)) = pq[i];
        }
        if (tid < kCsRows) lst[buf][tid] = ps;
    };
    float cs[kCsKT] = {};
    gload();
    lstore(0);
    if (nsteps > 1) gload();
    int rb = r0;  // rows of the step computed
    for (int s = 0; s < nsteps; s++) {
        __syncthreads();  // step s is in LDS; every wave is done with step s - 1
        if (s + 1 < nsteps) lstore((s + 1) & 1);
        if (s + 2 < nsteps) gload();
        const uint16_t *L = lq + (s & 1) * kCsBuf;
#pragma unroll
        for (int u = 0; u < kCsRows / 16; u++) {
            const int i0 = rb + 16 * u;
            if (i0 + 15 < jw) continue;  // rows before every key of this wave
            u4_t aq[4];
#pragma unroll
            for (int m = 0; m < 4; m++)
                aq[m] = *reinterpret_cast<const u4_t *>(L + (16 * u + r) * kKRow + 32 * m + 8 * kb);
            float st[4];
#pragma unroll
            for (int e = 0; e < 4; e++) st[e] = lst[s & 1][16 * u + 4 * kb + e];
            // the mask matters only where a key passes a row or rows pass T
            if (i0 < jw + 16 * kCsKT - 1 || i0 + 15 >= T)
                tile_colsum<DT, true>(aq, bk, st, cs, i0, jw, T, qscale, r, kb);
            else
                tile_colsum<DT, false>(aq, bk, st, cs, i0, jw, T, qscale, r, kb);
        }
        rb += kCsRows;
        if (rb >= r1) rb = r0;
    }
#pragma unroll
    for (int kt = 0; kt < kCsKT; kt++) {
        const float v = xrow_sum(cs[kt]);
        const int j = jw + 16 * kt + r;
        if (kb == 0 && j < T) dst[j] = v;
    }
}

// score[h][j] = sum of the chunks' partial sums, chunk 0 first
__global__ __launch_bounds__(256) void colsum_reduce_kernel(const float *__restrict__ part,
                                                            float *__restrict__ score, int T,
                                                            int cr, int nchunk) {
    const int h = blockIdx.y, j = blockIdx.x * 256 + threadIdx.x;
    if (j >= T) return;
    // chunks before c0 hold no row at or after the key block of j
    const int c0 = kCsKeys * (j / kCsKeys) / cr;
    float s = 0.0f;
    for (int c = c0; c < nchunk; c++) s += part[((size_t)h * nchunk + c) * T + j];
    score[(size_t)h * T + j] = s;
}

// ---------------------------------------------------------------- stage 3
// inclusive scan of v over the workgroup (thread order); *total = the sum.
// Wave scans, then a scan of the wave totals.
__device__ __forceinline__ unsigned block_scan(unsigned v, unsigned *wtot, unsigned *total) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const unsigned x = __shfl_up(v, off, 64);
        if (lane >= off) v += x;
    }
    if (lane == 63) wtot[w] = v;
    __syncthreads();
    if (w == 0) {
        unsigned s = lane < kSelThreads / 64 ? wtot[lane] : 0u;
#pragma unroll
        for (int off = 1; off < kSelThreads / 64; off <<= 1) {
            const unsigned x = __shfl_up(s, off, 64);
            if (lane >= off) s += x;
        }
        if (lane < kSelThreads / 64) wtot[lane] = s;
    }
    __syncthreads();
    const unsigned inc = v + (w > 0 ? wtot[w - 1] : 0u);
    *total = wtot[kSelThreads / 64 - 1];
    __syncthreads();
    return inc;
}

// One workgroup per KV head.  The heavy-th largest score among the positions
// before the window is found by a radix select over the fp32 bits (scores are
// >= 0, so the bits order like the values), 8 bits per pass with a 256-bin
// histogram in LDS; the positions at that score are then kept lowest first,
// and the kept positions are compacted in ascending order.
__global__ __launch_bounds__(kSelThreads) void select_kernel(const float *__restrict__ score,
                                                             int T, int heavy, int recent,
                                                             int32_t *__restrict__ keep,
                                                             int n_keep) {
    __shared__ unsigned hist[256];
    __shared__ unsigned wtot[kSelThreads / 64];
    __shared__ unsigned pick[2];
    __shared__ uint32_t cache[kSelCache];
    const int h = blockIdx.x, t = threadIdx.x;
    const uint32_t *sb = reinterpret_cast<const uint32_t *>(score + (size_t)h * T);
    // scores of up to kSelCache positions are read once into LDS
    const bool cached = T <= kSelCache;
    if (cached) {
        for (int x = t; x < T; x += kSelThreads) cache[x] = sb[x];
        __syncthreads();
    }
    auto bits = [&](int x) { return cached ? cache[x] : sb[x]; };
    const int rec = min(recent, T), n_old = T - rec, hv = min(heavy, n_old);
    const int chunk = (T + kSelThreads - 1) / kSelThreads;
    const int b0 = min(T, t * chunk), b1 = min(T, b0 + chunk), ob1 = min(n_old, b1);
    unsigned thr = 0xffffffffu, need = 0, tot;
    if (hv > 0) {
        unsigned prefix = 0, mask = 0;
        need = (unsigned)hv;  // rank of the wanted score among those matching the prefix
        for (int shift = 24; shift >= 0; shift -= 8) {
            if (t < 256) hist[t] = 0;
            __syncthreads();
            for (int x = b0; x < ob1; x++) {
                const uint32_t u = bits(x);
                if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
            }
            __syncthreads();
            // the first wave finds the bin holding the need-th largest: lane l
            // holds bins 255 - 4 l - [0, 4), the counts above it by a wave scan
            if (t < 64) {
                unsigned c[4], s4 = 0;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    c[e] = hist[255 - 4 * t - e];
                    s4 += c[e];
                }
                unsigned inc = s4;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const unsigned y = __shfl_up(inc, off, 64);
                    if (t >= off) inc += y;
                }
                unsigned above = inc - s4;  // in higher bins
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    if (above < need && above + c[e] >= need) {
                        pick[0] = 255u - 4 * t - e;
                        pick[1] = above;
                    }
                    above += c[e];
                }
            }
            __syncthreads();
            prefix |= pick[0] << shift;
            mask |= 255u << shift;
            need -= pick[1];
        }
        thr = prefix;  // the hv-th largest; need = how many at that score are kept
    }
    // ties at the threshold before this thread's chunk
    unsigned ties = 0;
    for (int x = b0; x < ob1; x++) ties += bits(x) == thr;
    const unsigned tie0 = block_scan(ties, wtot, &tot) - ties;
    // kept positions of this chunk, then their places
    unsigned kept = 0, rank = tie0;
    for (int x = b0; x < b1; x++) {
        const uint32_t u = bits(x);
        const bool k = x >= n_old || u > thr || (u == thr && rank++ < need);
        kept += k;
    }
    const unsigned pos0 = block_scan(kept, wtot, &tot) - kept;
    unsigned pos = pos0;
    rank = tie0;
    for (int x = b0; x < b1; x++) {
        const uint32_t u = bits(x);
        const bool k = x >= n_old || u > thr || (u == thr && rank++ < need);
        if (k && pos < (unsigned)n_keep) keep[(size_t)h * n_keep + pos++] = x;
    }
}

// ---------------------------------------------------------------- stage 4
// eight kept positions per workgroup: thread (row, K or V, 16-byte chunk)
__global__ __launch_bounds__(256) void gather_kernel(const uint16_t *__restrict__ k,
                                                     const uint16_t *__restrict__ v,
                                                     const int32_t *__restrict__ keep,
                                                     uint16_t *__restrict__ k_sel,
                                                     uint16_t *__restrict__ v_sel, int T,
                                                     int n_keep) {
    const int h = blockIdx.y, t = threadIdx.x, p = 8 * blockIdx.x + (t >> 5);
    if (p >= n_keep) return;
    const int src = min(max(keep[(size_t)h * n_keep + p], 0), T - 1);
    const int c8 = t & 15;
    const bool isk = (t & 16) == 0;
    const uint16_t *from = (isk ? k : v) + ((size_t)h * T + src) * D;
    uint16_t *to = (isk ? k_sel : v_sel) + ((size_t)h * n_keep + p) * D;
    *reinterpret_cast<uint4 *>(to + 8 * c8) = *reinterpret_cast<const uint4 *>(from + 8 * c8);
}

template <int DT>
hipError_t prefill_launch(const PrefillArgs &a, hipStream_t st) {
    const int g = a.Hq / a.Hkv;
    const float qscale = a.scale * kLog2e;
    hipLaunchKernelGGL(v_transpose_kernel, dim3(a.T32 / 32, a.Hkv), dim3(256), 0, st, a.v, a.vt,
                       a.T, a.T32);
    const int hw = g % 4 == 0 ? 4 : g % 2 == 0 ? 2 : 1;
    // with timing events: the dispatch's own start and end timestamps
    hipExtLaunchKernelGGL((prefill_fwd_kernel<DT>),
                          dim3(a.Hq / hw, (a.T + 128 / hw - 1) / (128 / hw), a.nsplit), dim3(256),
                          0, st, a.ev_before, a.ev_after, 0, a.q, a.k, (const uint16_t *)a.vt,
                          a.out, a.lse, a.T, a.T32, g, hw, qscale, a.kbc, a.nsplit, a.pml, a.pacc);
    if (a.nsplit > 1) {
        const int rows = a.Hq * a.T;
        hipLaunchKernelGGL(prefill_merge_kernel, dim3((rows + 3) / 4), dim3(256), 0, st, a.pml,
                           a.pacc, a.out, a.lse, a.T, rows, a.nsplit, a.kbc);
    }
    // query chunks of cr rows (a multiple of kCsRows), at most kColsumChunks of them
    const int cr = ((a.T + kColsumChunks - 1) / kColsumChunks + kCsRows - 1) / kCsRows * kCsRows;
    const int nchunk = (a.T + cr - 1) / cr;
    int n_cs = 0;
    for (int y = 0; y < nchunk; y++) n_cs += cs_blocks(y, cr, a.T);
    hipLaunchKernelGGL((prefill_colsum_kernel<DT>), dim3(n_cs, a.Hkv), dim3(256), 0, st, a.q, a.k,
                       a.lse, a.part, a.T, g, qscale, cr, nchunk);
    hipLaunchKernelGGL(colsum_reduce_kernel, dim3((a.T + 255) / 256, a.Hkv), dim3(256), 0, st,
                       a.part, a.score, a.T, cr, nchunk);
    if (a.n_keep > 0) {
        hipLaunchKernelGGL(select_kernel, dim3(a.Hkv), dim3(kSelThreads), 0, st, a.score, a.T,
                           a.heavy, a.recent, a.keep, a.n_keep);
        if (a.k_sel && a.v_sel)
            hipLaunchKernelGGL(gather_kernel, dim3((a.n_keep + 7) / 8, a.Hkv), dim3(256), 0, st,
                               a.k, a.v, a.keep, a.k_sel, a.v_sel, a.T, a.n_keep);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(int dtype, const PrefillArgs &a, hipStream_t st) {
    return dtype == F16 ? prefill_launch<F16>(a, st) : prefill_launch<BF16>(a, st);
}

}  // namespace kvq
