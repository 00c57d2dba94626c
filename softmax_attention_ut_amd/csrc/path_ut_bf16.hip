// path_ut (bf16 mode): per-chunk UT transform on gfx950 MFMA.
//
// Same quantities as the fp32 kernel in path_ut.hip (Chinese notes,
// training strategy: prod H = I - W^T T^{-1} W with
// T^{-1} = (I + strictLower(D W W^T))^{-1} D; Dutch summary section 3:
// boundary-adjusted keys computed per block beforehand), for chunks of
// C = 64 tokens and d in {64, 128}:
//     U  = T^{-1} W,   Y = T^{-1} strictLower(W K^T),   K~ = K - Y^T W,
//     Z  = T^{-T} W   (key-cache hand-off only)
// written in the operand layouts the scan kernel reads (see path_internal.h;
// permk = the k-slot permutation, applied to token axes and to the d rows of
// the transposed tiles):
//     kt [Lp][D]   K~ rows, natural
//     ut [N][D][C] -U^T:  ut[rho][sigma] = -U[permk(sigma)][permk(rho)]
//     vt [N][D][C]  V^T:  vt[rho][sigma] =  V[permk(sigma)][permk(rho)]
//                  (d = 128 only: the d = 64 scan reads V as it is with
//                  transpose loads)
//     yt [N][C][C]  Y^T:  yt[j][sigma]   =  Y[permk(sigma)][j]
//     zt [N][D][C] -Z^T, laid out like ut (key-cache hand-off only)
//     mt [N][D][D] -M^T with M = W^T U (the chunk's product is I - M in
//                  row-vector form): mt[rho][d'] = -M[d'][permk(rho)]
//                  (optional; the forward scan carries queries with it)
// plus the chunk-local forget-gate sums.
//
// The forward instances (DIAG) also take each query chunk's step with its own
// chunk (phase 4 below) and write the carried query, the pending
// probabilities and their maximum and sum instead of ut and yt.
//
// Arithmetic.  G = W W^T and R = W K^T are bf16 MFMAs with fp32
// accumulation (exact products of the bf16 inputs).  T^{-1} =
// (I + strictLower(D G))^{-1} D is formed in fp32, blocked by 16: the four
// diagonal 16-blocks by forward substitution (one lane per column,
//     X[m][n] = beta_m (delta_mn - sum_{p<m} G[m][p] X[p][n]),
// four blocks at once on one wave), the off-diagonal blocks from 16x16x4
// fp32 MFMA products of the blocks already known.  Products with the fp32
// factors T^{-1}, R and Y use a two-term bf16 split x = hi + lo
// (hi = bf16(x), lo = bf16(x - hi)), so they carry ~16 significant bits
// before the final bf16 rounding of the stored result.
#include "path_internal.h"

#include <type_traits>

namespace path {

namespace {

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16f(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void split8(const f32x16& acc, int half, float sign, bf16x8& hi,
                                       bf16x8& lo) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const float x = sign * acc[8 * half + t];
        const bf16 h = static_cast<bf16>(x);
        hi[t] = h;
        lo[t] = static_cast<bf16>(x - static_cast<float>(h));
    }
}

__device__ __forceinline__ bf16x8 ld8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ void zero(f32x16& a) {
#pragma unroll
    for (int v = 0; v < 16; ++v) a[v] = 0.f;
}

// bf16x8 from 8 consecutive accumulator registers, scaled
__device__ __forceinline__ bf16x8 cvt8(const f32x16& acc, int half, float sign) {
    bf16x8 r;
#pragma unroll
    for (int t = 0; t < 8; ++t) r[t] = static_cast<bf16>(sign * acc[8 * half + t]);
    return r;
}

// max / sum of a value with the lane 32 positions away (the two lane halves
// hold the two key halves of one query column)
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace

// Three workgroups per CU where LDS allows it (d = 64 without Z: 46 KB, held
// to 136 VGPRs by the bound); the other instances need more LDS per workgroup.
//
// DIAG (forward): the chunk's own-chunk step of the scan is taken here too,
// for its 64 queries (phase 4 below): the query carried to the chunk start and
// the probabilities of the chunk's own keys, with their maximum and sum.  U
// and Y then stay on chip (they serve no other step).
template <int D, bool WITH_Z, bool DIAG>
__global__ __launch_bounds__(256, (D == 64 && !WITH_Z) ? 3 : ((DIAG || WITH_Z) ? 2 : 1)) void path_ut_bf16_kernel(const UtArgs a) {
    static_assert(!DIAG || !WITH_Z, "the own-chunk step is a forward stage");
    constexpr int C = 64;
    constexpr int PW = D + 8;     // pitch of [token][d] tiles
    constexpr int PT = C + 8;     // pitch of [x][token-slot] bf16 tiles
    constexpr int GP = C + 8;     // pitch of the fp32 G rows (the T^{-1} hi/lo tiles reuse them)
    constexpr int ET = D / 32;
    constexpr int KSD = D / 16;

    __shared__ __attribute__((aligned(16))) bf16 sW[C * PW];     // W rows, d natural
    __shared__ __attribute__((aligned(16))) bf16 sK[C * PW];     // K rows
    __shared__ __attribute__((aligned(16))) bf16 sWt[D * PT];    // W^T: [rho][sigma] = W[permk(sigma)][permk(rho)]
    constexpr bool VT = D != 64 && !WITH_Z;  // V^T tiles are written (d = 128 forward)
    // G rows (p < m used), then X^T over its upper triangle (fp32); once X is
    // complete the same space holds T^{-1} rows with n in slots, hi and lo
    // (2 x C x PT bf16 = C x GP fp32)
    static_assert(2 * PT * 2 == GP * 4, "T^{-1} hi/lo tiles fill the G tile");
    __shared__ __attribute__((aligned(16))) float sG[C * GP];
    // V rows (d = 128 forward) are staged in the G tile: they are written out
    // as V^T before phase 1 forms G there
    static_assert(!VT || C * PW * 2 <= C * GP * 4, "V rows fit in the G tile");
    bf16* const sV = reinterpret_cast<bf16*>(sG);
    bf16* const sTh = reinterpret_cast<bf16*>(sG);
    bf16* const sTl = reinterpret_cast<bf16*>(sG) + C * PT;
    // T^{-T} rows, m slots, hi and lo.  d = 128 (ZK): formed after phase 3
    // over the K rows, which are no longer read then, as unpadded 64-wide rows
    // with their 16-byte units XOR-swizzled (so LDS fits two workgroups per CU)
    constexpr bool ZK = WITH_Z && D == 128;
    static_assert(!ZK || 2 * C * C <= C * PW, "the T^{-T} tiles fit over the K rows");
    __shared__ __attribute__((aligned(16))) bf16 sZh_[(WITH_Z && !ZK) ? C * PT : 8];
    __shared__ __attribute__((aligned(16))) bf16 sZl_[(WITH_Z && !ZK) ? C * PT : 8];
    bf16* const sZh = ZK ? sK : sZh_;
    bf16* const sZl = ZK ? sK + C * C : sZl_;
    // 16-byte unit u of T^{-T} row r
    auto zunit = [&](bf16* t, int r, int u) -> bf16* {
        return ZK ? t + r * C + ((u ^ ((r ^ (r >> 3)) & 7)) << 3) : t + r * PT + 8 * u;
    };
    __shared__ float sB[C];
    __shared__ __attribute__((aligned(16))) float sLoc[DIAG ? C : 4];   // -local log2 gate prefix (0 without gate)

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int L = a.L, N = a.N, Lp = N * C;
    const int head = blockIdx.x / N, c = blockIdx.x % N;
    const int p0 = c * C;
    const int nvalid = min(C, L - p0);
    const size_t rowbase = (size_t)head * Lp + p0;
    const size_t chunkbase = (size_t)head * N + c;

    float lf_in = 0.f;
    // DIAG: the queries of phase 4 (wave w: rows 32 (w & 1) .. +31, as the
    // B operand of k-step ks: d = 16 ks + 8 hh .. +7), loaded with the stage
    // (a load issued later would be waited for behind phase 3's stores)
    bf16x8 qv[KSD];
    if (DIAG) {
        const int iq = 32 * (wave & 1) + l32;
        const bf16* qrow = static_cast<const bf16*>(a.q) + ((size_t)head * L + p0 + iq) * D;
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
            qv[ks] = bf16x8{};
            if (iq < nvalid) qv[ks] = ld8(qrow + 16 * ks + 8 * hh);
        }
    }
    // ---- phase 0: stage W, K (rows), W^T (token slots), beta.  Every load
    // is issued before the first LDS write, so the stage waits for memory
    // once. ----
    {
        const bf16* w = static_cast<const bf16*>(a.w) + ((size_t)head * L + p0) * D;
        const bf16* k = static_cast<const bf16*>(a.k) + ((size_t)head * L + p0) * D;
        const bf16* v = static_cast<const bf16*>(a.v) + ((size_t)head * L + p0) * D;
        constexpr int UPR = D / 8;
        constexpr int NU = C * UPR / 256;          // 16-byte units per thread
        bf16x8 wv[NU], kv[NU], vv[NU];
#pragma unroll
        for (int it = 0; it < NU; ++it) {
            const int u = tid + 256 * it, r = u / UPR, d0 = (u % UPR) * 8;
            wv[it] = kv[it] = vv[it] = bf16x8{};
            if (r < nvalid) {
                wv[it] = ld8(w + (size_t)r * D + d0);
                kv[it] = ld8(k + (size_t)r * D + d0);
                if (VT) vv[it] = ld8(v + (size_t)r * D + d0);
            }
        }
        const float bta = (tid < C && tid < nvalid) ? a.beta[(size_t)head * L + p0 + tid] : 0.f;
        // wave 1's log f for the gate terms (phase 2), loaded with the rest
        if (wave == 1 && a.loc) lf_in = lane < nvalid ? a.log_f[(size_t)head * L + p0 + lane] : 0.f;
#pragma unroll
        for (int it = 0; it < NU; ++it) {
            const int u = tid + 256 * it, r = u / UPR, d0 = (u % UPR) * 8;
            *reinterpret_cast<bf16x8*>(sW + r * PW + d0) = wv[it];
            *reinterpret_cast<bf16x8*>(sK + r * PW + d0) = kv[it];
            if (VT) *reinterpret_cast<bf16x8*>(sV + r * PW + d0) = vv[it];
            const int slot = permk(r);
#pragma unroll
            for (int e = 0; e < 8; ++e) sWt[permk(d0 + e) * PT + slot] = wv[it][e];
        }
        if (tid < C) sB[tid] = bta;
    }
    __syncthreads();
    if constexpr (VT) {
        // V^T tile, 8 token slots per 16-byte store, out of the staged rows
        bf16* vt = static_cast<bf16*>(a.vt) + chunkbase * D * C;
#pragma unroll
        for (int it = 0; it < D * (C / 8) / 256; ++it) {
            const int u = tid + 256 * it;
            const int rho = u / (C / 8), s0 = (u % (C / 8)) * 8;
            const int e = permk(rho);
            bf16x8 col;
#pragma unroll
            for (int t = 0; t < 8; ++t) col[t] = sV[permk(s0 + t) * PW + e];
            *reinterpret_cast<bf16x8*>(vt + (size_t)rho * C + s0) = col;
        }
        __syncthreads();
    }

    // ---- phase 1: G tiles (m-block >= p-block), accumulator rows p, cols m ----
    if (wave < 3) {
        const int mb = wave == 0 ? 0 : 1, pb = wave == 2 ? 1 : 0;
        f32x16 g;
        zero(g);
        const bf16* ap = sW + (32 * pb + l32) * PW + 8 * hh;
        const bf16* bp = sW + (32 * mb + l32) * PW + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) g = mfma(ld8(ap + 16 * ks), ld8(bp + 16 * ks), g);
        float* grow = sG + (32 * mb + l32) * GP + 32 * pb + 4 * hh;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            f32x4 v4 = {g[4 * r4], g[4 * r4 + 1], g[4 * r4 + 2], g[4 * r4 + 3]};
            *reinterpret_cast<f32x4*>(grow + 8 * r4) = v4;
        }
    }
    __syncthreads();

    // ---- phase 2: X = T^{-1}, blocked by 16 ----
    // X is lower triangular.  X^T is written over the upper triangle of sG
    // (row n, columns m >= n hold X[m][n]); G below the diagonal stays where
    // the off-diagonal products need it.  The diagonal 16-blocks are stored
    // whole, zeros above their diagonal.
    //   (a) diagonal blocks X_bb = (I + strictLower(D_b G_bb))^{-1} D_b by
    //       forward substitution, four blocks at once on wave 0;
    //   (b) X_10, X_32 = -X_ii G_{i,i-1} X_{i-1,i-1};
    //   (c) the lower-left 32-block, -X'_11 G'_10 X'_00 over 32-blocks;
    // (I + A)^{-1} for the 2 x 2 block lower triangular I + A is
    // [[X0, 0], [-X1 A10 X0, X1]], and D A10 = D G10 puts the right-hand
    // diagonal into X1.
    if (wave == 0) {
        const int base = 16 * (lane >> 4), n = lane & 15;
        float t[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const float* grow = sG + (base + m) * GP + base;
            float acc = 0.f;
#pragma unroll
            for (int p = 0; p < m; ++p) acc = fmaf(grow[p], t[p], acc);
            t[m] = sB[base + m] * ((n == m ? 1.f : 0.f) - acc);
        }
        float* xrow = sG + (base + n) * GP + base;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<f32x4*>(xrow + 4 * q) = f32x4{t[4 * q], t[4 * q + 1], t[4 * q + 2], t[4 * q + 3]};
    } else {
        if (DIAG && wave == 1 && !a.loc) sLoc[lane] = 0.f;
        if (wave == 1 && a.loc) {
            // forget gate: chunk-local suffix sums in log2 units, fp64.  Lane s
            // holds log2 f_s; an inclusive suffix scan over the 64 lanes gives
            // x_s = sum_{s' >= s}, so loc_s = -(x_s - log2 f_s), csum = x_0.
            const double lf = lane < nvalid ? (double)lf_in * 1.4426950408889634 : 0.0;
            double x = lf;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const double y = __shfl_down(x, off, 64);
                if (lane + off < 64) x += y;
            }
            const float loc = static_cast<float>(-(x - lf));
            a.loc[rowbase + lane] = loc;
            if (DIAG) sLoc[lane] = loc;
            if (lane == 0) a.csum[chunkbase] = static_cast<float>(x);
            if (a.gb) {
                // the key's gate term -loc as the A row of the scan's bias
                // k-step: three bf16 terms, three ones, zeros
                const float g = -loc;
                const bf16 h = static_cast<bf16>(g);
                const float r = g - static_cast<float>(h);
                const bf16 m = static_cast<bf16>(r);
                const bf16 l = static_cast<bf16>(r - static_cast<float>(m));
                const bf16 one = static_cast<bf16>(1.f), nil = static_cast<bf16>(0.f);
                bf16x8* row = reinterpret_cast<bf16x8*>(static_cast<bf16*>(a.gb) + (rowbase + lane) * 16);
                row[0] = bf16x8{h, m, l, one, one, one, nil, nil};
                row[1] = bf16x8{nil, nil, nil, nil, nil, nil, nil, nil};
            }
        }
    }
    __syncthreads();

    // (b), (c): 16 x 16 x 4 fp32 MFMAs.  Lane l = 16 g + r; A supplies
    // A[r][k], B supplies B[k][r], and accumulator register v holds
    // row 4 g + v, column r.  The k index of step s is taken as 4 g + s, so an
    // accumulator feeds the next product's B operand register by register.
    {
        const int r = lane & 15, g = lane >> 4;
        if (wave < 2) {
            const int i = 2 * wave + 1, j = i - 1;
            const f32x4 a4 = *reinterpret_cast<const f32x4*>(sG + (16 * i + r) * GP + 16 * j + 4 * g);
            const f32x4 b4 = *reinterpret_cast<const f32x4*>(sG + (16 * j + r) * GP + 16 * j + 4 * g);
            f32x4 pacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 4; ++q) pacc = mfma16f(a4[q], b4[q], pacc);
            f32x4 xacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 4; ++q) xacc = mfma16f(sG[(16 * i + 4 * g + q) * GP + 16 * i + r], pacc[q], xacc);
            *reinterpret_cast<f32x4*>(sG + (16 * j + r) * GP + 16 * i + 4 * g) = -xacc;
        }
        __syncthreads();
        // (c): wave (rb, cb) forms the output 16-tile rows 32 + 16 rb, columns
        // 16 cb; it needs the 16-tiles (pb, cb), pb <= rb, of P = G'_10 X'_00.
        {
            const int rb = wave >> 1, cb = wave & 1;
            f32x4 pt[2];
#pragma unroll
            for (int pb = 0; pb < 2; ++pb) {
                pt[pb] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (pb > rb) continue;
                for (int kb = cb; kb < 2; ++kb) {  // X'_00[k][n] = 0 for k < n
                    const f32x4 a4 = *reinterpret_cast<const f32x4*>(sG + (32 + 16 * pb + r) * GP + 16 * kb + 4 * g);
                    const f32x4 b4 = *reinterpret_cast<const f32x4*>(sG + (16 * cb + r) * GP + 16 * kb + 4 * g);
#pragma unroll
                    for (int q = 0; q < 4; ++q) pt[pb] = mfma16f(a4[q], b4[q], pt[pb]);
                }
            }
            f32x4 xacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int pb = 0; pb < 2; ++pb) {
                if (pb > rb) continue;  // X'_11[r][c] = 0 for c > r
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    xacc = mfma16f(sG[(32 + 16 * pb + 4 * g + q) * GP + 32 + 16 * rb + r], pt[pb][q], xacc);
            }
            *reinterpret_cast<f32x4*>(sG + (16 * cb + r) * GP + 32 + 16 * rb + 4 * g) = -xacc;
        }
    }
    __syncthreads();

    // T^{-1} rows with the n axis in k-slot order, split hi/lo; for the key
    // cache also T^{-T} rows with the m axis in slot order.  X is read into
    // registers first: the hi/lo tiles overwrite it.
    static_assert(C * (C / 8) == 2 * 256, "two 8-slot units per thread");
    float xs[2][8], zs[2][8];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int u = tid + 256 * it, row = u >> 3, s0 = (u & 7) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int col = permk(s0 + e);
            xs[it][e] = col <= row ? sG[col * GP + row] : 0.f;
            if (WITH_Z) zs[it][e] = col >= row ? sG[row * GP + col] : 0.f;
        }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int u = tid + 256 * it, row = u >> 3, s0 = (u & 7) * 8;
        bf16x8 hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            hi[e] = static_cast<bf16>(xs[it][e]);
            lo[e] = static_cast<bf16>(xs[it][e] - static_cast<float>(hi[e]));
        }
        *reinterpret_cast<bf16x8*>(sTh + row * PT + s0) = hi;
        *reinterpret_cast<bf16x8*>(sTl + row * PT + s0) = lo;
        if (WITH_Z) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                hi[e] = static_cast<bf16>(zs[it][e]);
                lo[e] = static_cast<bf16>(zs[it][e] - static_cast<float>(hi[e]));
            }
            if (!ZK) {
                *reinterpret_cast<bf16x8*>(zunit(sZh, row, s0 >> 3)) = hi;
                *reinterpret_cast<bf16x8*>(zunit(sZl, row, s0 >> 3)) = lo;
            }
        }
    }
    __syncthreads();
    // Z[n][e] = sum_m T^{-1}[m][n] W[m][e] for the columns e of W^T row tile et
    auto zpart = [&](int et) {
        const int e = 32 * et + l32;         // W^T row rho: d = permk(rho)
        const bf16* bw = sWt + e * PT + 8 * hh;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            f32x16 zacc;
            zero(zacc);
#pragma unroll
            for (int ks = 2 * nt; ks < 4; ++ks) {   // T^{-T}[n][m] = 0 for m < n
                const bf16x8 w8 = ld8(bw + 16 * ks);
                zacc = mfma(ld8(zunit(sZh, 32 * nt + l32, 2 * ks + hh)), w8, zacc);
                zacc = mfma(ld8(zunit(sZl, 32 * nt + l32, 2 * ks + hh)), w8, zacc);
            }
            bf16* zrow = static_cast<bf16*>(a.zt) + (chunkbase * D + e) * C;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
                *reinterpret_cast<bf16x8*>(zrow + 32 * nt + 16 * s2 + 8 * hh) = cvt8(zacc, s2, -1.f);
        }
    };

    // ---- phase 3 ----
    // DIAG: the Y^T rows (waves 0, 1) and -U^T rows (waves 2, 3: d / 64 row
    // tiles each) are kept in registers for phase 4 instead of being stored.
    bf16x8 keep[D / 16];
    // R, Y and T^{-1} are triangular: tiles and k-steps that only meet their
    // zero blocks are skipped (key tile jt is wave-uniform, a compile-time
    // case each).
    auto keys = [&](auto jtc) {
        constexpr int jt = decltype(jtc)::value;   // key tile: columns j = 32 jt + l32
        const int j = 32 * jt + l32;
        // R[n][j] = w_n . k_j for n > j (accumulator rows n, cols j); the row
        // tile above the key tile (n < 32 jt) is zero
        f32x16 racc[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            zero(racc[nb]);
            if (nb < jt) continue;
            const bf16* ap = sW + (32 * nb + l32) * PW + 8 * hh;
            const bf16* bp = sK + j * PW + 8 * hh;
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) racc[nb] = mfma(ld8(ap + 16 * ks), ld8(bp + 16 * ks), racc[nb]);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int nrow = 32 * nb + 8 * (v >> 2) + 4 * hh + (v & 3);
                if (nrow <= j) racc[nb][v] = 0.f;
            }
        }
        bf16x8 rh[4], rl[4];
#pragma unroll
        for (int ks = 2 * jt; ks < 4; ++ks) split8(racc[ks >> 1], ks & 1, 1.f, rh[ks], rl[ks]);
        // Y[m][j] = sum_{j < n <= m} T^{-1}[m][n] R[n][j]: zero for m < 32 jt,
        // and k-steps n in [32 jt, 32 mb + 31]
        f32x16 yacc[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            zero(yacc[mb]);
            if (mb < jt) continue;
            const bf16* th = sTh + (32 * mb + l32) * PT + 8 * hh;
            const bf16* tl = sTl + (32 * mb + l32) * PT + 8 * hh;
#pragma unroll
            for (int ks = 2 * jt; ks < 2 * mb + 2; ++ks) {
                const bf16x8 ah = ld8(th + 16 * ks), al = ld8(tl + 16 * ks);
                yacc[mb] = mfma(ah, rh[ks], yacc[mb]);
                yacc[mb] = mfma(ah, rl[ks], yacc[mb]);
                yacc[mb] = mfma(al, rh[ks], yacc[mb]);
            }
        }
        // store Y^T[j][m-slot] (DIAG: keep it for phase 4)
        bf16* yrow = (DIAG || WITH_Z) ? nullptr : static_cast<bf16*>(a.yt) + (chunkbase * C + j) * C;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                if (DIAG) keep[2 * mb + s2] = cvt8(yacc[mb], s2, -1.f);   // -Y^T
                else if (!WITH_Z) *reinterpret_cast<bf16x8*>(yrow + 32 * mb + 16 * s2 + 8 * hh) = cvt8(yacc[mb], s2, 1.f);
            }
        // K~^T[d][j] = K^T[d][j] - sum_{m > j} W^T[d][m] Y[m][j]
        bf16x8 yh[4], yl[4];
#pragma unroll
        for (int ks = 2 * jt; ks < 4; ++ks) split8(yacc[ks >> 1], ks & 1, -1.f, yh[ks], yl[ks]);
        bf16* krow = static_cast<bf16*>(a.kt) + (rowbase + j) * D;
#pragma unroll
        for (int et = 0; et < ET; ++et) {
            // accumulator rows are sWt rows rho, i.e. d = permk(rho): register
            // 8s+t holds d = 32 et + 16 s + 8 hh + t
            f32x16 kacc;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const bf16x8 k8 = ld8(sK + j * PW + 32 * et + 16 * s2 + 8 * hh);
#pragma unroll
                for (int t = 0; t < 8; ++t) kacc[8 * s2 + t] = static_cast<float>(k8[t]);
            }
            const bf16* aw = sWt + (32 * et + l32) * PT + 8 * hh;
#pragma unroll
            for (int ks = 2 * jt; ks < 4; ++ks) {
                const bf16x8 w8 = ld8(aw + 16 * ks);
                kacc = mfma(w8, yh[ks], kacc);
                kacc = mfma(w8, yl[ks], kacc);
            }
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
                *reinterpret_cast<bf16x8*>(krow + 32 * et + 16 * s2 + 8 * hh) = cvt8(kacc, s2, 1.f);
        }
    };
    if (wave < 2) {
        if (__builtin_amdgcn_readfirstlane(wave) == 0) keys(std::integral_constant<int, 0>{});
        else keys(std::integral_constant<int, 1>{});
    } else {
        // waves 2, 3: U (and Z) for every token, a subset of the d columns
#pragma unroll
        for (int ei = 0; ei < ET / 2; ++ei) {
            const int et = wave - 2 + 2 * ei;
            const int e = 32 * et + l32;         // sWt row rho: d = permk(rho)
            const bf16* bw = sWt + e * PT + 8 * hh;
            // U[m][e] = sum_n T^{-1}[m][n] W[n][e]  (not needed by the hand-off)
            f32x16 uacc[2];
#pragma unroll
            for (int mt = 0; mt < 2 && !WITH_Z; ++mt) {
                zero(uacc[mt]);
                const bf16* th = sTh + (32 * mt + l32) * PT + 8 * hh;
                const bf16* tl = sTl + (32 * mt + l32) * PT + 8 * hh;
#pragma unroll
                for (int ks = 0; ks < 2 * mt + 2; ++ks) {   // T^{-1}[m][n] = 0 for n > m
                    const bf16x8 w8 = ld8(bw + 16 * ks);
                    uacc[mt] = mfma(ld8(th + 16 * ks), w8, uacc[mt]);
                    uacc[mt] = mfma(ld8(tl + 16 * ks), w8, uacc[mt]);
                }
            }
            bf16* urow = (DIAG || WITH_Z) ? nullptr : static_cast<bf16*>(a.ut) + (chunkbase * D + e) * C;
#pragma unroll
            for (int mt = 0; mt < 2 && !WITH_Z; ++mt)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    if (DIAG) keep[4 * ei + 2 * mt + s2] = cvt8(uacc[mt], s2, -1.f);
                    else *reinterpret_cast<bf16x8*>(urow + 32 * mt + 16 * s2 + 8 * hh) = cvt8(uacc[mt], s2, -1.f);
                }
            if (!WITH_Z && a.mt) {
                // M = W^T U (d x d): the whole chunk's transition product is
                // I - M in row-vector form.  The U accumulator's column is
                // d = permk(e), which is row e of -M^T in the stored layout
                // (row rho holds d = permk(rho)); columns d' come out natural.
                bf16x8 uh[4], ul[4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) split8(uacc[ks >> 1], ks & 1, 1.f, uh[ks], ul[ks]);
                bf16* mrow = static_cast<bf16*>(a.mt) + (chunkbase * D + e) * D;
#pragma unroll
                for (int ot = 0; ot < ET; ++ot) {
                    f32x16 macc;
                    zero(macc);
                    const bf16* aw = sWt + (32 * ot + l32) * PT + 8 * hh;
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const bf16x8 w8 = ld8(aw + 16 * ks);
                        macc = mfma(w8, uh[ks], macc);
                        macc = mfma(w8, ul[ks], macc);
                    }
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2)
                        *reinterpret_cast<bf16x8*>(mrow + 32 * ot + 16 * s2 + 8 * hh) = cvt8(macc, s2, -1.f);
                }
            }
            if (WITH_Z && !ZK) zpart(et);
        }
    }
    if constexpr (ZK) {
        // the T^{-T} tiles over the K rows (read by phase 3 until here), then
        // Z on all four waves, one W^T row tile each
        __syncthreads();
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int u = tid + 256 * it, row = u >> 3, s0 = (u & 7) * 8;
            bf16x8 hi, lo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                hi[e] = static_cast<bf16>(zs[it][e]);
                lo[e] = static_cast<bf16>(zs[it][e] - static_cast<float>(hi[e]));
            }
            *reinterpret_cast<bf16x8*>(zunit(sZh, row, s0 >> 3)) = hi;
            *reinterpret_cast<bf16x8*>(zunit(sZl, row, s0 >> 3)) = lo;
        }
        __syncthreads();
        zpart(wave);
    }
    if constexpr (DIAG) {
        // ---- phase 4: the chunk's own-chunk step for its 64 queries ----
        // (Chinese notes, training strategy: the full-matrix form of a block;
        // Dutch summary section 3: boundary-adjusted queries.)  For query i and
        // key j <= i of the chunk, with X = Q W^T:
        //     S = Q K^T - lower(X) Y          (= Q K~^T + strictUpper(X) Y)
        //     q~ = q - lower(X) U             (query carried to the chunk start)
        // in the scan's transposed orientation (S^T = K Q^T - Y^T lower(X)^T,
        // q~^T = Q^T + (-U^T) lower(X)^T), lower(X)^T coming out of the X^T
        // accumulator as the B operand over m.  Y^T and -U^T go over the T^{-1}
        // tiles (d = 128: -U^T fills both, Y^T goes over the W^T tile), which
        // are no longer read.
        bf16* const sUt = sTh;                     // -U^T rows rho, m in slots
        bf16* const sYt = D == 64 ? sTl : sWt;     // -Y^T rows j, m in slots
        __syncthreads();
        {
            auto put = [&](bf16* dst, int i) {
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2)
                        *reinterpret_cast<bf16x8*>(dst + 32 * b + 16 * s2 + 8 * hh) = keep[4 * i + 2 * b + s2];
            };
            if (wave < 2) {
                put(sYt + (32 * wave + l32) * PT, 0);
            } else {
#pragma unroll
                for (int ei = 0; ei < ET / 2; ++ei) put(sUt + (32 * (wave - 2 + 2 * ei) + l32) * PT, ei);
            }
        }
        __syncthreads();
        // wave w: query tile QT = w & 1 (rows 32 QT .. +31), role w >> 1 (0: the
        // probabilities, 1: the carried query).  Rows m (and keys j) of the
        // tiles above the query tile meet only the zero part of lower(X) (and
        // the mask), so those products are skipped: a compile-time case each.
        auto own = [&](auto qtc, auto rolec) {
            constexpr int QT = decltype(qtc)::value, ROLE = decltype(rolec)::value;
            constexpr int KM = 2 * (QT + 1);        // k-steps over m that meet lower(X)
            const int iloc = 32 * QT + l32;
            const size_t row = rowbase + iloc;
            f32x16 x[2];
#pragma unroll
            for (int kt2 = 0; kt2 <= QT; ++kt2) {
                zero(x[kt2]);
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks)
                    x[kt2] = mfma(ld8(sW + (32 * kt2 + l32) * PW + 16 * ks + 8 * hh), qv[ks], x[kt2]);
            }
            // lower(X)^T: rows m <= i
            bf16x8 xl[KM];
#pragma unroll
            for (int ks = 0; ks < KM; ++ks)
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int v = 8 * (ks & 1) + t;
                    const int m = 32 * (ks >> 1) + 8 * (v >> 2) + 4 * hh + (v & 3);
                    xl[ks][t] = static_cast<bf16>(m <= iloc ? x[ks >> 1][v] : 0.f);
                }
            if constexpr (ROLE == 0) {
                // S^T = K Q^T + (-Y^T) lower(X)^T for key tiles kt2 <= QT
                f32x16 s[2];
#pragma unroll
                for (int kt2 = 0; kt2 <= QT; ++kt2) {
                    zero(s[kt2]);
#pragma unroll
                    for (int ks = 0; ks < KSD; ++ks)
                        s[kt2] = mfma(ld8(sK + (32 * kt2 + l32) * PW + 16 * ks + 8 * hh), qv[ks], s[kt2]);
#pragma unroll
                    for (int ks = 0; ks < KM; ++ks)
                        s[kt2] = mfma(ld8(sYt + (32 * kt2 + l32) * PT + 16 * ks + 8 * hh), xl[ks], s[kt2]);
                }
                // z = scale log2(e) S + log2 prod_{s=j+1}^{i} f_s  (= loc_i - loc_j,
                // zero without the gate), causal mask j <= i (key tile QT only);
                // lane: keys j = 32 kt2 + 8 (v/4) + 4 hh + v%4, four consecutive
                // per group
                const float li = sLoc[iloc];
                float mx = -INFINITY;
#pragma unroll
                for (int kt2 = 0; kt2 <= QT; ++kt2)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x4 lj = *reinterpret_cast<const f32x4*>(sLoc + 32 * kt2 + 8 * g + 4 * hh);
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const int v = 4 * g + c;
                            const int j = 32 * kt2 + 8 * g + 4 * hh + c;
                            float z = fmaf(s[kt2][v], a.scale2, li - lj[c]);
                            if (kt2 == QT && j > iloc) z = -INFINITY;
                            s[kt2][v] = z;
                            mx = fmaxf(mx, z);
                        }
                    }
                mx = pair_max(mx);
                // probabilities as the scan's PV B operand: register ks holds the
                // accumulator registers 8 (ks & 1) .. +7 of key tile ks >> 1 (zero
                // above the query tile); the row sum is taken over the rounded
                // values the PV product uses
                const bf16x2 ones = {static_cast<bf16>(1.f), static_cast<bf16>(1.f)};
                float psum = 0.f;
                bf16* prow = static_cast<bf16*>(a.pd) + row * C;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    bf16x8 p8 = {};
                    if ((ks >> 1) <= QT) {
#pragma unroll
                        for (int t = 0; t < 8; ++t)
                            p8[t] = static_cast<bf16>(__builtin_amdgcn_exp2f(s[ks >> 1][8 * (ks & 1) + t] - mx));
#pragma unroll
                        for (int t = 0; t < 8; t += 2)
                            psum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p8[t], p8[t + 1]}, ones, psum, false);
                    }
                    *reinterpret_cast<bf16x8*>(prow + 16 * ks + 8 * hh) = p8;
                }
                psum = pair_sum(psum);
                if (hh == 0) *reinterpret_cast<f32x2*>(a.ml + 2 * row) = f32x2{mx, psum};
            } else {
                // q~^T = Q^T + (-U^T) lower(X)^T, then times scale log2(e)
                f32x16 qacc[ET];
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks)
#pragma unroll
                    for (int t = 0; t < 8; ++t) qacc[ks >> 1][8 * (ks & 1) + t] = static_cast<float>(qv[ks][t]);
#pragma unroll
                for (int dt = 0; dt < ET; ++dt)
#pragma unroll
                    for (int ks = 0; ks < KM; ++ks)
                        qacc[dt] = mfma(ld8(sUt + (32 * dt + l32) * PT + 16 * ks + 8 * hh), xl[ks], qacc[dt]);
                // register 8 s + t of tile dt holds d = 32 dt + 16 s + 8 hh + t
                bf16* qrow = static_cast<bf16*>(a.qt) + row * D;
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks)
                    *reinterpret_cast<bf16x8*>(qrow + 16 * ks + 8 * hh) = cvt8(qacc[ks >> 1], ks & 1, a.scale2);
            }
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        switch (__builtin_amdgcn_readfirstlane(wave)) {
            case 0: own(I0{}, I0{}); break;
            case 1: own(I1{}, I0{}); break;
            case 2: own(I0{}, I1{}); break;
            default: own(I1{}, I1{}); break;
        }
    }
}

hipError_t launch_path_ut_bf16(const UtArgs& a, hipStream_t s) {
    const dim3 grid(a.BH * a.N), block(256);
    const bool z = a.zt != nullptr;
    if (a.D == 64) {
        if (z) hipLaunchKernelGGL((path_ut_bf16_kernel<64, true, false>), grid, block, 0, s, a);
        else if (a.qt) hipLaunchKernelGGL((path_ut_bf16_kernel<64, false, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((path_ut_bf16_kernel<64, false, false>), grid, block, 0, s, a);
    } else if (a.D == 128) {
        if (z) hipLaunchKernelGGL((path_ut_bf16_kernel<128, true, false>), grid, block, 0, s, a);
        else if (a.qt) hipLaunchKernelGGL((path_ut_bf16_kernel<128, false, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((path_ut_bf16_kernel<128, false, false>), grid, block, 0, s, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace path
