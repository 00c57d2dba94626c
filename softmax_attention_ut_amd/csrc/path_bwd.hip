// path_bwd: gradients of the PaTH(-FoX) attention forward (gfx950), bf16
// inputs, d = 64, chunks of C = 64 tokens.
//
// The pages say that training uses the same blockwise algorithm as the
// forward (English summary; Dutch summary section 3); the backward here is
// the exact gradient of that algorithm, read back through each of its steps
// (Chinese notes, training strategy: the UT transform, the full-matrix form
// of a block and the right-to-left transport).  Per head, with the forward's
// per-chunk quantities (T^{-1}, U = T^{-1} W, Y = T^{-1} strictLower(W K^T),
// K~ = K - Y^T W, M = W^T U, chunk c's whole product P_c = I - M_c in
// row-vector form) and, for query chunk a and key chunk b < a,
//     Q_{a,a-1} = Q~_a = Q_a - lower(Q_a W_a^T) U_a,
//     Q_{a,b-1} = Q_{a,b} P_b,
//     S_ab = scale Q_{a,b} K~_b^T + (F_i - F_j),
//     S_aa = scale (Q_a K_a^T - lower(Q_a W_a^T) Y_a) + (F_i - F_j), j <= i,
// softmax rows P = exp(S - lse), dP = dO V^T, dS = P (dP - rowsum(dO o O)):
//   * dV_b = sum_a P_ab^T dO_a,  dK~_b = scale sum_a dS_ab^T Q_{a,b};
//   * the query's adjoint runs left to right: G_0 = dQ_{a,0},
//     G_b = dQ_{a,b} + G_{b-1} P_b^T, dQ_{a,b} = scale dS_ab K~_b, and the
//     chunk product gets dM_b = -sum_a Q_{a,b}^T G_{a,b-1}; dQ~_a = G_{a-1};
//   * the own chunk and the carry to its start give dQ_a, dK_a, dW_a, dU_a,
//     dY_a directly;
//   * the UT transform of each chunk turns dK~, dY, dU, dM into dK, dW and
//     dbeta (through T^{-1} = (I + strictLower(D W W^T))^{-1} D);
//   * the gate: F_i - F_j gives dF = rowsum(dS) - colsum(dS) per token and
//     dlog f_t = sum_{i >= t} dF_i.
//
// Kernels (after the forward's prepare stage, path_ut_bf16, for K~, U, Y, M
// and the gate sums):
//   path_bwd_query_kernel  one workgroup per (head, query chunk a): the own
//       chunk, then Q_{a,b} right to left (stored per pair), then the adjoint
//       G left to right (stored per pair), then dQ~_a and dQ_a;
//   path_bwd_key_kernel    one workgroup per (head, key chunk b): the sums over
//       the query chunks a > b, then the chunk's UT-transform backward;
//   path_bwd_gate_kernel   one workgroup per head: dlog f by suffix sums.
// Every 64 x 64 x 64 product is four bf16 MFMAs per wave (32 x 32 quarter
// tiles, fp32 accumulation) on LDS tiles; the stored per-pair states
// (Q_{a,b}, G_{a,b-1}) are bf16.
#include "path_internal.h"

namespace path {

namespace {

constexpr int BC = 64;        // chunk = head dim
constexpr int BP = BC + 8;    // LDS tile pitch (bf16 elements)
constexpr int BT = BC * BP;   // LDS tile size (elements)
constexpr int FP = BC + 1;    // fp32 LDS tile pitch

__device__ __forceinline__ f32x16 mfmab(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 l8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f32x16 z16() {
    f32x16 z;
#pragma unroll
    for (int v = 0; v < 16; ++v) z[v] = 0.f;
    return z;
}

// Wave w owns the 32 x 32 quarter (rows 32 (w >> 1) .., cols 32 (w & 1) ..)
// of a 64 x 64 result; register v of lane l holds row qrow(w, l, v), column
// qcol(w, l) (the 32x32x16 MFMA accumulator layout).
__device__ __forceinline__ int qrow(int wave, int lane, int v) {
    return 32 * (wave >> 1) + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}
__device__ __forceinline__ int qcol(int wave, int lane) { return 32 * (wave & 1) + (lane & 31); }

// acc += A B^T over k = 0..63: out[m][n] = sum_k A[m][k] B[n][k], both bf16
// LDS tiles [64][BP] (16-byte operand reads).
__device__ __forceinline__ f32x16 mm_nt(const bf16* A, const bf16* B, f32x16 acc, int wave, int lane) {
    const int l32 = lane & 31, hh = lane >> 5;
    const bf16* ar = A + (32 * (wave >> 1) + l32) * BP + 8 * hh;
    const bf16* br = B + (32 * (wave & 1) + l32) * BP + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = mfmab(l8(ar + 16 * ks), l8(br + 16 * ks), acc);
    return acc;
}

// quarter -> bf16 LDS tile, as is ([m][n]) or transposed ([n][m]), times s
template <bool TR>
__device__ __forceinline__ void st_q(bf16* T, const f32x16& acc, int wave, int lane, float s = 1.f) {
    const int n = qcol(wave, lane);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int m = qrow(wave, lane, v);
        const bf16 x = static_cast<bf16>(s * acc[v]);
        if (TR) T[n * BP + m] = x;
        else T[m * BP + n] = x;
    }
}
// quarter -> fp32 global [64][64] (rows of 64 floats), added to what is there when ADD
template <bool ADD>
__device__ __forceinline__ void st_qg(float* G, const f32x16& acc, int wave, int lane, float s = 1.f) {
    const int n = qcol(wave, lane);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int m = qrow(wave, lane, v);
        if (ADD) G[m * BC + n] += s * acc[v];
        else G[m * BC + n] = s * acc[v];
    }
}
__device__ __forceinline__ f32x16 ld_qg(const float* G, int wave, int lane) {
    const int n = qcol(wave, lane);
    f32x16 r;
#pragma unroll
    for (int v = 0; v < 16; ++v) r[v] = G[qrow(wave, lane, v) * BC + n];
    return r;
}

// Row-major [rows][64] bf16 global rows -> LDS tile, as is or transposed;
// rows >= nvalid are zero.  256 threads, 16-byte units.
template <bool TR>
__device__ __forceinline__ void ld_tile(bf16* T, const bf16* g, int nvalid, int tid) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int u = tid + 256 * it, r = u >> 3, c0 = (u & 7) * 8;
        bf16x8 x = {};
        if (r < nvalid) x = l8(g + (size_t)r * BC + c0);
        if (TR) {
#pragma unroll
            for (int e = 0; e < 8; ++e) T[(c0 + e) * BP + r] = x[e];
        } else {
            *reinterpret_cast<bf16x8*>(T + r * BP + c0) = x;
        }
    }
}
// fp32 [64][64] global -> bf16 LDS tile (as is or transposed), times s
template <bool TR>
__device__ __forceinline__ void ld_tile_f(bf16* T, const float* g, int tid, float s = 1.f) {
    for (int u = tid; u < BC * BC; u += 256) {
        const int r = u >> 6, c = u & 63;
        const bf16 x = static_cast<bf16>(s * g[u]);
        if (TR) T[c * BP + r] = x;
        else T[r * BP + c] = x;
    }
}

// The forward's stored chunk tiles (path_ut_bf16 layouts, permk = the k-slot
// permutation) -> natural or transposed bf16 LDS tiles.
//   ut[rho][sigma] = -U[permk(sigma)][permk(rho)]
//   yt[j][sigma]   =  Y[permk(sigma)][j]
//   mt[rho][e]     = -M[e][permk(rho)]
// U_NAT: T[m][e] = U[m][e];  U_TR: T[e][m] = U[m][e]
template <bool TR>
__device__ __forceinline__ void ld_u(bf16* T, const bf16* ut, int tid) {
    for (int u = tid; u < BC * BC; u += 256) {
        const int rho = u >> 6, sig = u & 63;
        const bf16 x = static_cast<bf16>(-static_cast<float>(ut[u]));
        const int m = permk(sig), e = permk(rho);
        if (TR) T[e * BP + m] = x;
        else T[m * BP + e] = x;
    }
}
// Y_NAT: T[m][j] = Y[m][j];  Y_TR: T[j][m] = Y[m][j]
template <bool TR>
__device__ __forceinline__ void ld_y(bf16* T, const bf16* yt, int tid) {
    for (int u = tid; u < BC * BC; u += 256) {
        const int j = u >> 6, sig = u & 63;
        const int m = permk(sig);
        if (TR) T[j * BP + m] = yt[u];
        else T[m * BP + j] = yt[u];
    }
}
// M_NAT: T[x][y] = M[x][y];  M_TR: T[y][x] = M[x][y]
template <bool TR>
__device__ __forceinline__ void ld_m(bf16* T, const bf16* mt, int tid) {
    for (int u = tid; u < BC * BC; u += 256) {
        const int rho = u >> 6, e = u & 63;
        const bf16 x = static_cast<bf16>(-static_cast<float>(mt[u]));
        const int y = permk(rho);      // M[e][y]
        if (TR) T[y * BP + e] = x;
        else T[e * BP + y] = x;
    }
}

__device__ __forceinline__ float wave_sum32(float x) {   // over the 32 lanes of a half
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) x += __shfl_xor(x, off, 32);
    return x;
}

// index of the pair (a, b), b < a, in the per-head pair arrays
__device__ __forceinline__ size_t pair_index(int a, int b) { return (size_t)a * (a - 1) / 2 + b; }

}  // namespace

// Workspace sections of the backward (set up by the API layer).
// Per head: pairs = N (N - 1) / 2.
//   qs, gs   [BH][pairs][64][64] bf16   Q_{a,b} and G_{a,b-1} (b >= 1)
//   own      [BH][N][5][64][64] fp32     per chunk: dK (own-chunk step),
//                                        dV (own chunk), dY, dU, dW (own chunk)
//   dsum     [BH][Lp] fp32   rowsum(dO o O) per query
//   rsum     [BH][Lp] fp32   rowsum(dS) per query (all its keys)
//   csd      [BH][Lp] fp32   colsum(dS) of the own-chunk step per key
//   csl      [BH][Lp] fp32   colsum(dS) over the later query chunks per key
using BwdKArgs = BwdArgs;

// ---------------------------------------------------------------------------
// Query-stationary: one workgroup (4 waves) per (head, query chunk a).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void path_bwd_query_kernel(const BwdKArgs a) {
    __shared__ __attribute__((aligned(16))) bf16 tA[BT], tB[BT], tCt[BT], tD[BT], tE[BT],
        tF[BT], tH[BT], tI[BT], tJ[BT], tXl[BT], tXlT[BT];
    __shared__ float sLse[BC], sD[BC], sLoc[BC], sLocK[BC], sRow[BC], sCol[BC];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int L = a.L, N = a.N, Lp = N * BC;
    const int head = blockIdx.x / N, ca = blockIdx.x % N;
    const int p0 = ca * BC, nva = min(BC, L - p0);
    const size_t hrow = (size_t)head * L;      // input rows of the head
    const size_t wrow = (size_t)head * Lp;     // workspace rows of the head
    const bool gate = a.loc != nullptr;
    const float c2 = a.scale * kLog2e;
    const int n = qcol(wave, lane);

    const bf16* q = static_cast<const bf16*>(a.q) + (hrow + p0) * BC;
    const bf16* k = static_cast<const bf16*>(a.k) + (hrow + p0) * BC;
    const bf16* vv = static_cast<const bf16*>(a.v);
    const bf16* w = static_cast<const bf16*>(a.w) + (hrow + p0) * BC;
    const bf16* o = static_cast<const bf16*>(a.out) + (hrow + p0) * BC;
    const bf16* dO = static_cast<const bf16*>(a.dout) + (hrow + p0) * BC;
    const bf16* ktw = static_cast<const bf16*>(a.kt) + wrow * BC;
    const bf16* mtw = static_cast<const bf16*>(a.mt) + (size_t)head * N * BC * BC;
    float* own = a.own + ((size_t)head * N + ca) * 5 * BC * BC;

    // rowsum(dO o O), lse, gate terms
    if (tid < BC) {
        float s = 0.f;
        if (tid < nva)
            for (int e = 0; e < BC; ++e)
                s += static_cast<float>(dO[(size_t)tid * BC + e]) * static_cast<float>(o[(size_t)tid * BC + e]);
        sD[tid] = s;
        a.dsum[wrow + p0 + tid] = s;
        sLse[tid] = tid < nva ? a.lse[hrow + p0 + tid] * kLog2e : 0.f;
        sLoc[tid] = gate ? a.loc[wrow + p0 + tid] : 0.f;
        sRow[tid] = 0.f;
        sCol[tid] = 0.f;
    }
    // ---- own chunk: S = scale (Q K^T - lower(X) Y) + gate, X = Q W^T ----
    ld_tile<false>(tA, q, nva, tid);         // Q
    ld_tile<false>(tB, w, nva, tid);         // W
    ld_tile<false>(tCt, k, nva, tid);        // K
    ld_y<true>(tD, static_cast<const bf16*>(a.yt) + ((size_t)head * N + ca) * BC * BC, tid);   // Y^T [j][m]
    ld_tile<false>(tE, dO, nva, tid);        // dO
    ld_tile<false>(tF, vv + (hrow + p0) * BC, nva, tid);   // V (own)
    __syncthreads();
    f32x16 x = mm_nt(tA, tB, z16(), wave, lane);            // X[i][m]
#pragma unroll
    for (int v = 0; v < 16; ++v)
        if (n > qrow(wave, lane, v)) x[v] = 0.f;            // lower: m <= i
    st_q<false>(tXl, x, wave, lane);
    st_q<true>(tXlT, x, wave, lane);
    __syncthreads();
    f32x16 s = mm_nt(tA, tCt, z16(), wave, lane);           // Q K^T
    f32x16 xy = mm_nt(tXl, tD, z16(), wave, lane);          // lower(X) Y
    f32x16 dp = mm_nt(tE, tF, z16(), wave, lane);           // dO V^T
    f32x16 ds, pp;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int i = qrow(wave, lane, v);
        const float z = c2 * (s[v] - xy[v]) + (sLoc[i] - sLoc[n]);
        const float p = (n <= i && i < nva) ? exp2f(z - sLse[i]) : 0.f;
        pp[v] = p;
        ds[v] = p * (dp[v] - sD[i]);
    }
    // gate sums of the own chunk
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const float r = wave_sum32(ds[v]);
        if ((lane & 31) == 0) atomicAdd(&sRow[qrow(wave, lane, v)], r);
    }
    {
        float cs = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) cs += ds[v];
        cs += __shfl_xor(cs, 32, 64);
        if (lane < 32) atomicAdd(&sCol[n], cs);
    }
    __syncthreads();                          // tile reads done; reuse tH, tI for dS, P
    st_q<false>(tH, ds, wave, lane);          // dS [i][j]
    st_q<true>(tI, ds, wave, lane);           // dS^T [j][i]
    st_q<true>(tJ, pp, wave, lane);           // P^T [j][i]
    // dO^T, Q^T for the own-chunk dV, dK
    ld_tile<true>(tD, dO, nva, tid);          // dO^T [d][i]   (Y^T no longer needed)
    ld_tile<true>(tF, q, nva, tid);           // Q^T [d][i]
    __syncthreads();
    // dV_own = P^T dO, dK_own = scale dS^T Q, dY = -scale lower(X)^T dS
    st_qg<false>(own + 1 * BC * BC, mm_nt(tJ, tD, z16(), wave, lane), wave, lane);
    st_qg<false>(own + 0 * BC * BC, mm_nt(tI, tF, z16(), wave, lane), wave, lane, a.scale);
    st_qg<false>(own + 2 * BC * BC, mm_nt(tXlT, tI, z16(), wave, lane), wave, lane, -a.scale);
    __syncthreads();                          // P^T, dO^T reads done
    // dQ (own chunk) = scale dS K:  K^T needed [d][j]
    ld_tile<true>(tJ, k, nva, tid);           // K^T [d][j]
    ld_y<false>(tD, static_cast<const bf16*>(a.yt) + ((size_t)head * N + ca) * BC * BC, tid);   // Y [m][j]
    __syncthreads();
    f32x16 dq = mm_nt(tH, tJ, z16(), wave, lane);           // dS K, unscaled
#pragma unroll
    for (int v = 0; v < 16; ++v) dq[v] *= a.scale;
    // dXl = -scale dS Y^T (lower)
    f32x16 dxl = mm_nt(tH, tD, z16(), wave, lane);
#pragma unroll
    for (int v = 0; v < 16; ++v) dxl[v] = (n <= qrow(wave, lane, v)) ? -a.scale * dxl[v] : 0.f;

    // ---- Q~ = Q - lower(X) U (the query carried to the chunk start) ----
    ld_u<true>(tE, static_cast<const bf16*>(a.ut) + ((size_t)head * N + ca) * BC * BC, tid);  // U^T [e][m]
    __syncthreads();
    f32x16 qc = mm_nt(tXl, tE, z16(), wave, lane);          // lower(X) U
    {
        // Q quarter: tA holds Q [i][d]
#pragma unroll
        for (int v = 0; v < 16; ++v) qc[v] = static_cast<float>(tA[qrow(wave, lane, v) * BP + n]) - qc[v];
    }
    // ---- right to left: Q_{a,b}, b = a-1 .. 0, stored ----
    bf16* qs = static_cast<bf16*>(a.qs) + (size_t)head * ((size_t)N * (N - 1) / 2) * BC * BC;
    bf16* gs = static_cast<bf16*>(a.gs) + (size_t)head * ((size_t)N * (N - 1) / 2) * BC * BC;
    for (int b = ca - 1; b >= 0; --b) {
        __syncthreads();
        st_q<false>(tB, qc, wave, lane);                    // Q_{a,b}
        if (b >= 1) ld_m<true>(tCt, mtw + (size_t)b * BC * BC, tid);   // M_b^T [y][x]
        __syncthreads();
        {
            bf16* dst = qs + pair_index(ca, b) * BC * BC;
            for (int u = tid; u < BC * BC / 8; u += 256) {
                const int r = u >> 3, c0 = (u & 7) * 8;
                *reinterpret_cast<bf16x8*>(dst + r * BC + c0) = l8(tB + r * BP + c0);
            }
        }
        if (b >= 1) {
            const f32x16 qm = mm_nt(tB, tCt, z16(), wave, lane);   // Q M_b
#pragma unroll
            for (int v = 0; v < 16; ++v) qc[v] -= qm[v];
        }
    }
    // ---- left to right: dS_ab, the adjoint G, dQ_{a,b} ----
    __syncthreads();                                         // U^T reads done
    ld_tile<false>(tE, dO, nva, tid);                        // dO [i][d]
    double fsum = 0.0;                                       // sum of csum over chunks b+1 .. a (log2)
    if (gate)
        for (int c = 1; c <= ca; ++c) fsum += static_cast<double>(a.csum[(size_t)head * N + c]);
    f32x16 g = z16();
    for (int b = 0; b < ca; ++b) {
        __syncthreads();
        ld_tile<false>(tA, qs + pair_index(ca, b) * BC * BC, BC, tid);   // Q_{a,b}
        ld_tile<false>(tCt, ktw + (size_t)b * BC * BC, BC, tid);         // K~_b
        ld_tile<true>(tD, ktw + (size_t)b * BC * BC, BC, tid);           // K~_b^T
        ld_tile<false>(tF, vv + (hrow + (size_t)b * BC) * BC, BC, tid);  // V_b (chunks left of a are full)
        if (gate && tid < BC) sLocK[tid] = a.loc[wrow + (size_t)b * BC + tid];
        if (b >= 1) ld_m<false>(tH, mtw + (size_t)b * BC * BC, tid);    // M_b [x][y]
        st_q<false>(tI, g, wave, lane);                                  // G_{b-1}
        __syncthreads();
        if (b >= 1) {
            bf16* dst = gs + pair_index(ca, b) * BC * BC;
            for (int u = tid; u < BC * BC / 8; u += 256) {
                const int r = u >> 3, c0 = (u & 7) * 8;
                *reinterpret_cast<bf16x8*>(dst + r * BC + c0) = l8(tI + r * BP + c0);
            }
        }
        const float bias_q = static_cast<float>(fsum);
        f32x16 sb = mm_nt(tA, tCt, z16(), wave, lane);       // Q_{a,b} K~_b^T
        f32x16 db = mm_nt(tE, tF, z16(), wave, lane);        // dO V_b^T
        f32x16 dsb;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int i = qrow(wave, lane, v);
            const float z = c2 * sb[v] + (gate ? sLoc[i] + bias_q - sLocK[n] : 0.f);
            const float p = i < nva ? exp2f(z - sLse[i]) : 0.f;
            dsb[v] = p * (db[v] - sD[i]);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float r = wave_sum32(dsb[v]);
            if ((lane & 31) == 0) atomicAdd(&sRow[qrow(wave, lane, v)], r);
        }
        f32x16 gm = z16();
        if (b >= 1) gm = mm_nt(tI, tH, z16(), wave, lane);   // G_{b-1} M_b^T
        __syncthreads();                                     // tH, tI reads done
        st_q<false>(tH, dsb, wave, lane);                    // dS [i][j]
        __syncthreads();
        const f32x16 dqb = mm_nt(tH, tD, z16(), wave, lane); // dS K~_b
#pragma unroll
        for (int v = 0; v < 16; ++v) g[v] = a.scale * dqb[v] + (b >= 1 ? g[v] - gm[v] : 0.f);
        if (gate) fsum -= static_cast<double>(a.csum[(size_t)head * N + b + 1]);
    }
    // ---- dQ~ = G_{a-1}: Q~ backward.  dQ += dQ~ ; dXl += -(dQ~ U^T) lower ;
    // dU = -lower(X)^T dQ~ ; then dQ += dXl W, dW_own = dXl^T Q ----
    __syncthreads();
    st_q<false>(tI, g, wave, lane);                          // dQ~ [i][e]
    st_q<true>(tH, g, wave, lane);                           // dQ~^T [e][i]
    ld_u<false>(tD, static_cast<const bf16*>(a.ut) + ((size_t)head * N + ca) * BC * BC, tid);  // U [m][e]
    ld_tile<true>(tCt, w, nva, tid);                         // W^T [d][m]
    ld_tile<true>(tF, q, nva, tid);                          // Q^T [d][i]
    __syncthreads();
    const f32x16 du = mm_nt(tI, tD, z16(), wave, lane);      // (dQ~ U^T)[i][m]
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        dq[v] += g[v];
        dxl[v] -= (n <= qrow(wave, lane, v)) ? du[v] : 0.f;
    }
    // dU = -lower(X)^T dQ~: rows m, cols e
    st_qg<false>(own + 3 * BC * BC, mm_nt(tXlT, tH, z16(), wave, lane), wave, lane, -1.f);
    __syncthreads();
    st_q<false>(tA, dxl, wave, lane);                        // dXl [i][m]
    st_q<true>(tB, dxl, wave, lane);                         // dXl^T [m][i]
    __syncthreads();
    const f32x16 dqw = mm_nt(tA, tCt, z16(), wave, lane);    // dXl W
    st_qg<false>(own + 4 * BC * BC, mm_nt(tB, tF, z16(), wave, lane), wave, lane);   // dW_own = dXl^T Q
    // final dQ rows of this chunk
    {
        float* dqg = a.dq + (hrow + p0) * BC;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int i = qrow(wave, lane, v);
            if (i < nva) dqg[(size_t)i * BC + n] = dq[v] + dqw[v];
        }
    }
    __syncthreads();
    if (tid < BC) {
        a.rsum[wrow + p0 + tid] = sRow[tid];
        a.csd[wrow + p0 + tid] = sCol[tid];
    }
}

// ---------------------------------------------------------------------------
// Key-stationary: one workgroup per (head, key chunk b): sums over the query
// chunks a > b, then the chunk's UT-transform backward.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void path_bwd_key_kernel(const BwdKArgs a) {
    __shared__ __attribute__((aligned(16))) bf16 tA[BT], tB[BT], tCt[BT], tD[BT], tE[BT],
        tF[BT], tH[BT], tI[BT];
    __shared__ float sG[BC * FP], sX[BC * FP];   // fp32: G, then (I + A)^{-1}
    __shared__ float sLse[BC], sD[BC], sLocQ[BC], sLocK[BC], sCol[BC], sB[BC], sDb[BC];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int L = a.L, N = a.N, Lp = N * BC;
    const int head = blockIdx.x / N, cb = blockIdx.x % N;
    const int p0 = cb * BC, nvb = min(BC, L - p0);
    const size_t hrow = (size_t)head * L, wrow = (size_t)head * Lp;
    const bool gate = a.loc != nullptr;
    const float c2 = a.scale * kLog2e;
    const int n = qcol(wave, lane);

    const bf16* vv = static_cast<const bf16*>(a.v);
    const bf16* dOg = static_cast<const bf16*>(a.dout);
    const bf16* ktw = static_cast<const bf16*>(a.kt) + wrow * BC;
    const bf16* qs = static_cast<const bf16*>(a.qs) + (size_t)head * ((size_t)N * (N - 1) / 2) * BC * BC;
    const bf16* gs = static_cast<const bf16*>(a.gs) + (size_t)head * ((size_t)N * (N - 1) / 2) * BC * BC;
    const float* own = a.own + ((size_t)head * N + cb) * 5 * BC * BC;

    ld_tile<false>(tA, ktw + (size_t)cb * BC * BC, BC, tid);         // K~_b [j][d]
    ld_tile<false>(tB, vv + (hrow + p0) * BC, nvb, tid);             // V_b [j][d]
    if (tid < BC) {
        sLocK[tid] = gate ? a.loc[wrow + p0 + tid] : 0.f;
        sCol[tid] = 0.f;
    }
    f32x16 dv = z16(), dkt = z16(), dm = z16();
    double fsum = 0.0;     // sum of csum over chunks b+1 .. a
    for (int ca = cb + 1; ca < N; ++ca) {
        const int pa = ca * BC, nva = min(BC, L - pa);
        if (gate) fsum += static_cast<double>(a.csum[(size_t)head * N + ca]);
        __syncthreads();
        const bf16* qab = qs + pair_index(ca, cb) * BC * BC;
        ld_tile<false>(tCt, qab, BC, tid);                           // Q_{a,b} [i][d]
        ld_tile<true>(tD, qab, BC, tid);                             // Q_{a,b}^T [d][i]
        ld_tile<false>(tE, dOg + (hrow + pa) * BC, nva, tid);        // dO_a [i][d]
        ld_tile<true>(tF, dOg + (hrow + pa) * BC, nva, tid);         // dO_a^T [d][i]
        if (cb >= 1) ld_tile<true>(tH, gs + pair_index(ca, cb) * BC * BC, BC, tid);   // G^T [y][i]
        if (tid < BC) {
            sLse[tid] = tid < nva ? a.lse[hrow + pa + tid] * kLog2e : 0.f;
            sD[tid] = a.dsum[wrow + pa + tid];
            sLocQ[tid] = gate ? a.loc[wrow + pa + tid] : 0.f;
        }
        __syncthreads();
        const float bias_q = static_cast<float>(fsum);
        const f32x16 sb = mm_nt(tCt, tA, z16(), wave, lane);         // Q K~^T [i][j]
        const f32x16 db = mm_nt(tE, tB, z16(), wave, lane);          // dO V^T [i][j]
        f32x16 pq, dsq;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int i = qrow(wave, lane, v);
            const float z = c2 * sb[v] + (gate ? sLocQ[i] + bias_q - sLocK[n] : 0.f);
            const float p = i < nva ? exp2f(z - sLse[i]) : 0.f;
            pq[v] = p;
            dsq[v] = p * (db[v] - sD[i]);
        }
        {
            float cs = 0.f;
#pragma unroll
            for (int v = 0; v < 16; ++v) cs += dsq[v];
            cs += __shfl_xor(cs, 32, 64);
            if (lane < 32) atomicAdd(&sCol[n], cs);
        }
        // P^T, dS^T as [j][i] tiles (over tE: dO rows are no longer needed)
        __syncthreads();
        st_q<true>(tE, pq, wave, lane);                              // P^T [j][i]
        st_q<true>(tI, dsq, wave, lane);                             // dS^T [j][i]
        __syncthreads();
        dv = mm_nt(tE, tF, dv, wave, lane);                          // P^T dO   [j][d]
        dkt = mm_nt(tI, tD, dkt, wave, lane);                        // dS^T Q   [j][d] (unscaled)
        if (cb >= 1) dm = mm_nt(tD, tH, dm, wave, lane);             // Q^T G    [x][y]
    }
    // ---- totals ----
    // dV = P^T dO (later queries) + own chunk
    {
        const f32x16 dvo = ld_qg(own + 1 * BC * BC, wave, lane);
        float* dvg = a.dv + (hrow + p0) * BC;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int j = qrow(wave, lane, v);
            if (j < nvb) dvg[(size_t)j * BC + n] = dv[v] + dvo[v];
        }
    }
    __syncthreads();
    if (tid < BC) a.csl[wrow + p0 + tid] = sCol[tid];
    // ---- UT-transform backward of chunk b ----
    // Inputs: dK~ = scale dkt, dM = -dm, and from the query side dU, dY and
    // the own-chunk dK, dW.  Recomputed: G = W W^T, X = (I + A)^{-1} with
    // A = strictLower(D G), T^{-1} = X D, R = strictLower(W K^T), Y = T^{-1} R,
    // U = T^{-1} W.  Tiles: tA W [m][e], tB W^T [e][m], tCt K [j][e],
    // tD K^T [e][j], tE T^{-1} [m][n], tF T^{-1}^T [n][m]; tH, tI scratch.
    const bf16* wg = static_cast<const bf16*>(a.w) + (hrow + p0) * BC;
    const bf16* kg = static_cast<const bf16*>(a.k) + (hrow + p0) * BC;
    __syncthreads();
    ld_tile<false>(tA, wg, nvb, tid);
    ld_tile<true>(tB, wg, nvb, tid);
    ld_tile<false>(tCt, kg, nvb, tid);
    ld_tile<true>(tD, kg, nvb, tid);
    if (tid < BC) {
        sB[tid] = tid < nvb ? a.beta[hrow + p0 + tid] : 0.f;
        sDb[tid] = 0.f;
    }
    __syncthreads();
    {
        const f32x16 gq = mm_nt(tA, tA, z16(), wave, lane);         // G = W W^T
#pragma unroll
        for (int v = 0; v < 16; ++v) sG[qrow(wave, lane, v) * FP + n] = gq[v];
    }
    __syncthreads();
    // X = (I + A)^{-1} (unit lower triangular) by forward substitution, four
    // lanes per column c: X[m][c] = delta_mc - beta_m sum_{c <= p < m} G[m][p] X[p][c]
    {
        const int col = tid >> 2, sp = tid & 3;
        for (int m = 0; m < BC; ++m) {
            float part = 0.f;
            for (int p = col + sp; p < m; p += 4) part += sG[m * FP + p] * sX[p * FP + col];
            part += __shfl_xor(part, 1, 4);
            part += __shfl_xor(part, 2, 4);
            if (sp == 0) sX[m * FP + col] = (m == col ? 1.f : 0.f) - (m > col ? sB[m] * part : 0.f);
            __syncthreads();
        }
    }
    for (int u = tid; u < BC * BC; u += 256) {                      // T^{-1} = X D
        const int m = u >> 6, c = u & 63;
        const bf16 t = static_cast<bf16>(sX[m * FP + c] * sB[c]);
        tE[m * BP + c] = t;
        tF[c * BP + m] = t;
    }
    __syncthreads();
    f32x16 rq = mm_nt(tA, tCt, z16(), wave, lane);                  // W K^T [n][j]
#pragma unroll
    for (int v = 0; v < 16; ++v)
        if (qrow(wave, lane, v) <= n) rq[v] = 0.f;                   // strictly lower: n > j
    const f32x16 uq = mm_nt(tE, tB, z16(), wave, lane);             // U = T^{-1} W [m][e]
    st_q<true>(tH, rq, wave, lane);                                  // R^T [j][n]
    __syncthreads();
    const f32x16 yq = mm_nt(tE, tH, z16(), wave, lane);             // Y = T^{-1} R [m][j]
    f32x16 dK = ld_qg(own + 0 * BC * BC, wave, lane);
    f32x16 dW = ld_qg(own + 4 * BC * BC, wave, lane);
    f32x16 dY = ld_qg(own + 2 * BC * BC, wave, lane);
    f32x16 dU = ld_qg(own + 3 * BC * BC, wave, lane);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        dkt[v] *= a.scale;                                           // dK~
        dK[v] += dkt[v];                                             // K~ = K - Y^T W
        dm[v] = -dm[v];                                              // dM
    }
    __syncthreads();
    st_q<false>(tH, dkt, wave, lane);                                // dK~ [j][e]
    st_q<true>(tI, dkt, wave, lane);                                 // dK~^T [e][j]
    __syncthreads();
    {
        const f32x16 t1 = mm_nt(tA, tH, z16(), wave, lane);         // W dK~^T [m][j]
#pragma unroll
        for (int v = 0; v < 16; ++v) dY[v] -= t1[v];
    }
    __syncthreads();
    st_q<false>(tCt, yq, wave, lane);                                // Y [m][j] (over K)
    __syncthreads();
    {
        const f32x16 t1 = mm_nt(tCt, tI, z16(), wave, lane);        // Y dK~ [m][e]
#pragma unroll
        for (int v = 0; v < 16; ++v) dW[v] -= t1[v];
    }
    // M = W^T U: dW += U dM^T, dU += W dM
    __syncthreads();
    st_q<false>(tH, uq, wave, lane);                                 // U [m][y]
    st_q<false>(tI, dm, wave, lane);                                 // dM [x][y]
    __syncthreads();
    {
        const f32x16 t1 = mm_nt(tH, tI, z16(), wave, lane);         // U dM^T [m][x]
#pragma unroll
        for (int v = 0; v < 16; ++v) dW[v] += t1[v];
    }
    __syncthreads();
    st_q<true>(tI, dm, wave, lane);                                  // dM^T [y][x]
    __syncthreads();
    {
        const f32x16 t1 = mm_nt(tA, tI, z16(), wave, lane);         // W dM [m][y]
#pragma unroll
        for (int v = 0; v < 16; ++v) dU[v] += t1[v];
    }
    // Y = T^{-1} R, U = T^{-1} W: dT^{-1} = dY R^T + dU W^T
    __syncthreads();
    st_q<false>(tH, dY, wave, lane);                                 // dY [m][j]
    st_q<false>(tI, rq, wave, lane);                                 // R [n][j]
    st_q<false>(tCt, dU, wave, lane);                                // dU [m][e]
    __syncthreads();
    f32x16 dT = mm_nt(tH, tI, z16(), wave, lane);                   // dY R^T [m][n]
    dT = mm_nt(tCt, tA, dT, wave, lane);                             // + dU W^T
    // dR = T^{-T} dY (strictly lower), dW += T^{-T} dU
    __syncthreads();
    st_q<true>(tH, dY, wave, lane);                                  // dY^T [j][m]
    st_q<true>(tI, dU, wave, lane);                                  // dU^T [e][m]
    __syncthreads();
    f32x16 dR = mm_nt(tF, tH, z16(), wave, lane);                   // [n][j]
#pragma unroll
    for (int v = 0; v < 16; ++v)
        if (qrow(wave, lane, v) <= n) dR[v] = 0.f;
    {
        const f32x16 t1 = mm_nt(tF, tI, z16(), wave, lane);         // T^{-T} dU [n][e]
#pragma unroll
        for (int v = 0; v < 16; ++v) dW[v] += t1[v];
    }
    // R = strictLower(W K^T): dW += dR K, dK += dR^T W
    __syncthreads();
    st_q<false>(tH, dR, wave, lane);                                 // dR [n][j]
    st_q<true>(tI, dR, wave, lane);                                  // dR^T [j][n]
    __syncthreads();
    {
        const f32x16 t1 = mm_nt(tH, tD, z16(), wave, lane);         // dR K [n][e]
        const f32x16 t2 = mm_nt(tI, tB, z16(), wave, lane);         // dR^T W [j][e]
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            dW[v] += t1[v];
            dK[v] += t2[v];
        }
    }
    // T^{-1} = X D: dX = dT^{-1} D, dbeta_c += sum_m X[m][c] dT^{-1}[m][c]
    f32x16 dX;
    {
        float cs = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int m = qrow(wave, lane, v);
            dX[v] = dT[v] * sB[n];
            cs += sX[m * FP + n] * dT[v];
        }
        cs += __shfl_xor(cs, 32, 64);
        if (lane < 32) atomicAdd(&sDb[n], cs);
    }
    // X = (I + A)^{-1}: dA = -X^T dX X^T via Z = dX X^T, dA = -X^T Z
    __syncthreads();
    st_q<false>(tH, dX, wave, lane);                                 // dX [m][c]
    for (int u = tid; u < BC * BC; u += 256) {
        const int m = u >> 6, c = u & 63;
        const bf16 x = static_cast<bf16>(sX[m * FP + c]);
        tI[m * BP + c] = x;                                          // X [p][c]
        tCt[c * BP + m] = x;                                         // X^T [c][m]
    }
    __syncthreads();
    const f32x16 zq = mm_nt(tH, tI, z16(), wave, lane);             // Z = dX X^T [m][p]
    __syncthreads();
    st_q<true>(tH, zq, wave, lane);                                  // Z^T [p][m]
    __syncthreads();
    f32x16 dA = mm_nt(tCt, tH, z16(), wave, lane);                  // X^T Z [q][p]
    // A = strictLower(D G): dbeta_q += sum_{p<q} dA[q][p] G[q][p], dG = beta_q dA
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int qr = qrow(wave, lane, v);
        const float da = (n < qr) ? -dA[v] : 0.f;
        dA[v] = sB[qr] * da;
        const float r = wave_sum32(da * sG[qr * FP + n]);
        if ((lane & 31) == 0) atomicAdd(&sDb[qr], r);
    }
    // G = W W^T: dW += (dG + dG^T) W
    __syncthreads();
    st_q<false>(tH, dA, wave, lane);                                 // dG [q][p]
    __syncthreads();
    for (int u = tid; u < BC * BC; u += 256) {
        const int r = u >> 6, c = u & 63;
        tI[r * BP + c] = static_cast<bf16>(static_cast<float>(tH[r * BP + c]) + static_cast<float>(tH[c * BP + r]));
    }
    __syncthreads();
    {
        const f32x16 t1 = mm_nt(tI, tB, z16(), wave, lane);         // (dG + dG^T) W [q][e]
#pragma unroll
        for (int v = 0; v < 16; ++v) dW[v] += t1[v];
    }
    __syncthreads();
    {
        float* dkg = a.dk + (hrow + p0) * BC;
        float* dwg = a.dw + (hrow + p0) * BC;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = qrow(wave, lane, v);
            if (r < nvb) {
                dkg[(size_t)r * BC + n] = dK[v];
                dwg[(size_t)r * BC + n] = dW[v];
            }
        }
        if (tid < nvb) a.dbeta[hrow + p0 + tid] = sDb[tid];
    }
}

// ---------------------------------------------------------------------------
// Gate: dF_t = rowsum_t - colsum_t, dlog f_t = sum_{i >= t} dF_i (one
// workgroup per head, fp64 run sums).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void path_bwd_gate_kernel(const BwdKArgs a) {
    __shared__ double sTot[256];
    const int head = blockIdx.x, tid = threadIdx.x;
    const int L = a.L, Lp = a.N * BC;
    const int run = (L + 255) / 256;
    const int r0 = min(tid * run, L), r1 = min(r0 + run, L);
    const size_t wrow = (size_t)head * Lp;
    auto df = [&](int t) {
        return static_cast<double>(a.rsum[wrow + t]) - static_cast<double>(a.csd[wrow + t]) -
               static_cast<double>(a.csl[wrow + t]);
    };
    double tot = 0.0;
    for (int t = r0; t < r1; ++t) tot += df(t);
    sTot[tid] = tot;
    __syncthreads();
    // exclusive suffix sums of the run totals
    for (int off = 1; off < 256; off <<= 1) {
        const double y = tid + off < 256 ? sTot[tid + off] : 0.0;
        __syncthreads();
        sTot[tid] += y;
        __syncthreads();
    }
    double acc = sTot[tid] - tot;                 // sum over runs after this one
    for (int t = r1 - 1; t >= r0; --t) {
        acc += df(t);
        a.dlogf[(size_t)head * L + t] = static_cast<float>(acc);
    }
}

hipError_t launch_path_bwd(const BwdArgs& a, hipStream_t s) {
    const dim3 grid(a.BH * a.N), block(256);
    hipLaunchKernelGGL(path_bwd_query_kernel, grid, block, 0, s, a);
    hipLaunchKernelGGL(path_bwd_key_kernel, grid, block, 0, s, a);
    if (a.log_f) hipLaunchKernelGGL(path_bwd_gate_kernel, dim3(a.BH), block, 0, s, a);
    return hipGetLastError();
}

}  // namespace path
