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
//     dlog f_t = sum_{i >= t} dF_i, i.e. the sum of dS over the block
//     i >= t, j < t.  The row sums vanish in exact arithmetic (sum_j dS_ij =
//     dO_i . O_i - D_i), but the computed ones carry the rounding of the
//     stored O in D_i, and keeping them makes the suffix sums equal that
//     block sum of the computed dS, whose keys j < t hold little of a
//     decaying row's weight; the column sums alone would give the
//     complementary block, where that rounding weighs most.
//
// Kernels (after the forward's prepare stage, path_ut_bf16, for K~, U, Y, M
// and the gate sums):
//   path_bwd_layout_kernel one workgroup per (head, chunk): U, Y, M from the
//       prepare stage's operand layouts to row-major tiles, in place;
//   path_bwd_query_kernel  one workgroup per (head, query chunk a): the own
//       chunk, then Q_{a,b} right to left (stored per pair), then the adjoint
//       G left to right (stored per pair), then dQ~_a and dQ_a;
//   path_bwd_key_kernel    one workgroup per (head, key chunk b): dV, dK~ and
//       dM summed over the query chunks a > b;
//   path_bwd_ut_kernel     one workgroup per (head, chunk): the chunk's
//       UT-transform backward -> dK, dW, dbeta;
//   path_bwd_gate_kernel   one workgroup per head: dlog f by suffix sums.
// Every 64 x 64 x 64 product is four bf16 MFMAs per wave (32 x 32 quarter
// tiles, fp32 accumulation) on LDS tiles; the stored per-pair states
// (Q_{a,b}, G_{a,b-1}) are bf16.  Global tiles move as 16-byte fragments,
// fetched for the next step of a loop while the current step computes; the
// query and key kernels keep eight LDS tiles (74 KB) so that two workgroups
// share a CU.
#include "path_internal.h"

namespace path {

namespace {

constexpr int BC = 64;        // chunk = head dim
constexpr int BP = BC + 8;    // LDS tile pitch (bf16 elements)
constexpr int BT = BC * BP;   // LDS tile size (elements)
constexpr int FP = BC + 4;    // fp32 LDS tile pitch (rows 16-byte aligned)
constexpr int NOWN = 9;       // fp32 64 x 64 partials per chunk (see below)

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
// quarter <-> fp32 global [64][64] (rows of 64 floats)
__device__ __forceinline__ void st_qg(float* G, const f32x16& acc, int wave, int lane, float s = 1.f) {
    const int n = qcol(wave, lane);
#pragma unroll
    for (int v = 0; v < 16; ++v) G[qrow(wave, lane, v) * BC + n] = s * acc[v];
}
__device__ __forceinline__ f32x16 ld_qg(const float* G, int wave, int lane) {
    const int n = qcol(wave, lane);
    f32x16 r;
#pragma unroll
    for (int v = 0; v < 16; ++v) r[v] = G[qrow(wave, lane, v) * BC + n];
    return r;
}

// A 64 x 64 bf16 tile of row-major [64][64] global rows in flight: thread t
// holds rows 2 (t & 31) and 2 (t & 31) + 1, columns 8 (t >> 5) .. + 7.  fetch
// issues the loads (rows >= nvalid read as zero); put / put_t write the
// fragment to an LDS tile as is or transposed (then each pair of rows is one
// 4-byte word per column: the 64 lanes of a wave hit 64 distinct banks).
struct Frag { bf16x8 x[2]; };
__device__ __forceinline__ Frag fetch(const bf16* g, int nvalid, int tid) {
    const int r = 2 * (tid & 31), c = 8 * (tid >> 5);
    const bf16x8 z = {};
    Frag f;
    f.x[0] = r < nvalid ? l8(g + (size_t)r * BC + c) : z;
    f.x[1] = r + 1 < nvalid ? l8(g + (size_t)(r + 1) * BC + c) : z;
    return f;
}
__device__ __forceinline__ void put(bf16* T, const Frag& f, int tid) {
    const int r = 2 * (tid & 31), c = 8 * (tid >> 5);
    *reinterpret_cast<bf16x8*>(T + r * BP + c) = f.x[0];
    *reinterpret_cast<bf16x8*>(T + (r + 1) * BP + c) = f.x[1];
}
__device__ __forceinline__ void put_t(bf16* T, const Frag& f, int tid) {
    const int r = 2 * (tid & 31), c = 8 * (tid >> 5);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const bf16x2 p = {f.x[0][e], f.x[1][e]};
        *reinterpret_cast<bf16x2*>(T + (c + e) * BP + r) = p;
    }
}
// LDS tile -> row-major [64][64] global rows (16-byte stores)
__device__ __forceinline__ void store_tile(bf16* g, const bf16* T, int tid) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int u = tid + 256 * it, r = u >> 3, c = (u & 7) * 8;
        *reinterpret_cast<bf16x8*>(g + r * BC + c) = l8(T + r * BP + c);
    }
}

__device__ __forceinline__ float wave_sum32(float x) {   // over the 32 lanes of a half
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) x += __shfl_xor(x, off, 32);
    return x;
}

// Workgroup -> (head, chunk).  Workgroups are dealt to the 8 XCDs in turn;
// when B*H is a multiple of 8, head h goes to XCD h % 8 and its chunks run
// together there, so the per-chunk tiles every chunk of a head reads (K~,
// V, M, d_out) stay in that XCD's L2.  rev: chunks in decreasing order.
__device__ __forceinline__ void wg_map(int x, int BH, int N, bool rev, int& head, int& c) {
    if ((BH & 7) == 0) {
        const int slot = x >> 3;
        head = (slot / N) * 8 + (x & 7);
        c = slot % N;
    } else {
        head = x / N;
        c = x % N;
    }
    if (rev) c = N - 1 - c;
}

// index of the pair (a, b), b < a, in the per-head pair arrays
__device__ __forceinline__ size_t pair_index(int a, int b) { return (size_t)a * (a - 1) / 2 + b; }

// sD[r] = rowsum(dO o O) of the 64 rows at dO, O (rows >= nvalid: 0), four
// threads per row
__device__ __forceinline__ void row_dots(float* sD, const bf16* dO, const bf16* O, int nvalid, int tid) {
    const int r = tid >> 2, c = 16 * (tid & 3);
    float s = 0.f;
    if (r < nvalid) {
        const bf16x8 a0 = l8(dO + (size_t)r * BC + c), a1 = l8(dO + (size_t)r * BC + c + 8);
        const bf16x8 b0 = l8(O + (size_t)r * BC + c), b1 = l8(O + (size_t)r * BC + c + 8);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            s += static_cast<float>(a0[e]) * static_cast<float>(b0[e]) +
                 static_cast<float>(a1[e]) * static_cast<float>(b1[e]);
    }
    s += __shfl_xor(s, 1, 4);
    s += __shfl_xor(s, 2, 4);
    if ((tid & 3) == 0) sD[r] = s;
}

}  // namespace

// Workspace sections of the backward (set up by the API layer).
// Per head: pairs = N (N - 1) / 2.
//   qs, gs   [BH][pairs][64][64] bf16   Q_{a,b} and G_{a,b-1} (b >= 1)
//   own      [BH][N][9][64][64] fp32     per chunk: dK (own-chunk step),
//                                        dV (own chunk), dY, dU, dW (own
//                                        chunk), dK~, dM, and the query
//                                        kernel's dQ and dX partials, held
//                                        there across its two loops
//   dsum     [BH][Lp] fp32   rowsum(dO o O) per query
//   rsum     [BH][Lp] fp32   rowsum(dS) per query (all its keys)
//   csd      [BH][Lp] fp32   colsum(dS) of the own-chunk step per key
//   csl      [BH][Lp] fp32   colsum(dS) over the later query chunks per key
// ut, yt, mt hold U, Y, M as row-major tiles once path_bwd_layout_kernel ran.
using BwdKArgs = BwdArgs;

// ---------------------------------------------------------------------------
// U, Y, M of one chunk from the prepare stage's operand layouts (permk = its
// k-slot permutation) to row-major tiles, in place:
//   ut[rho][sigma] = -U[permk(sigma)][permk(rho)]   -> U[m][e]
//   yt[j][sigma]   =  Y[permk(sigma)][j]            -> Y[m][j]
//   mt[rho][e]     = -M[e][permk(rho)]              -> M[x][y]
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void path_bwd_layout_kernel(const BwdKArgs a) {
    __shared__ __attribute__((aligned(16))) bf16 tU[BT], tY[BT], tM[BT];
    const int tid = threadIdx.x;
    const size_t base = (size_t)blockIdx.x * BC * BC;
    bf16* ut = static_cast<bf16*>(a.ut) + base;
    bf16* yt = static_cast<bf16*>(a.yt) + base;
    bf16* mt = static_cast<bf16*>(a.mt) + base;
    bf16 xu[16], xy[16], xm[16];
#pragma unroll
    for (int it = 0; it < 16; ++it) {
        const int u = tid + 256 * it;
        xu[it] = ut[u];
        xy[it] = yt[u];
        xm[it] = mt[u];
    }
#pragma unroll
    for (int it = 0; it < 16; ++it) {
        const int u = tid + 256 * it, hi = u >> 6, lo = u & 63;
        tU[permk(lo) * BP + permk(hi)] = static_cast<bf16>(-static_cast<float>(xu[it]));
        tY[permk(lo) * BP + hi] = xy[it];
        tM[lo * BP + permk(hi)] = static_cast<bf16>(-static_cast<float>(xm[it]));
    }
    __syncthreads();
    store_tile(ut, tU, tid);
    store_tile(yt, tY, tid);
    store_tile(mt, tM, tid);
}

// ---------------------------------------------------------------------------
// Query-stationary: one workgroup (4 waves) per (head, query chunk a).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 2) void path_bwd_query_kernel(const BwdKArgs a) {
    __shared__ __attribute__((aligned(16))) bf16 tA[BT], tB[BT], tC[BT], tD[BT], tE[BT], tF[BT],
        tX[BT], tXT[BT];
    __shared__ float sLse[BC], sD[BC], sLoc[BC], sLocK[BC], sRow[BC], sCol[BC];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int L = a.L, N = a.N, Lp = N * BC;
    int head, ca;
    wg_map(blockIdx.x, a.BH, N, true, head, ca);
    const int p0 = ca * BC, nva = min(BC, L - p0);
    const size_t hrow = (size_t)head * L;      // input rows of the head
    const size_t wrow = (size_t)head * Lp;     // workspace rows of the head
    const size_t chunk0 = (size_t)head * N;    // first chunk of the head
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
    const bf16* un = static_cast<const bf16*>(a.ut) + (chunk0 + ca) * BC * BC;
    const bf16* yn = static_cast<const bf16*>(a.yt) + (chunk0 + ca) * BC * BC;
    const bf16* mn = static_cast<const bf16*>(a.mt) + chunk0 * BC * BC;
    float* own = a.own + (chunk0 + ca) * NOWN * BC * BC;

    // ---- own chunk: S = scale (Q K^T - lower(X) Y) + gate, X = Q W^T ----
    Frag fq = fetch(q, nva, tid), fw = fetch(w, nva, tid), fk = fetch(k, nva, tid);
    const Frag fy = fetch(yn, BC, tid), fo = fetch(dO, nva, tid);
    const Frag fv = fetch(vv + (hrow + p0) * BC, nva, tid);
    Frag fu = fetch(un, BC, tid);
    row_dots(sD, dO, o, nva, tid);
    if (tid < BC) {
        sLse[tid] = tid < nva ? a.lse[hrow + p0 + tid] * kLog2e : 0.f;
        sLoc[tid] = gate ? a.loc[wrow + p0 + tid] : 0.f;
        sRow[tid] = 0.f;
        sCol[tid] = 0.f;
    }
    put(tA, fq, tid);          // Q [i][d]
    put(tB, fw, tid);          // W [m][d]
    put(tC, fk, tid);          // K [j][d]
    put_t(tD, fy, tid);        // Y^T [j][m]
    put(tE, fo, tid);          // dO [i][d]
    put(tF, fv, tid);          // V [j][d]
    __syncthreads();
    if (tid < BC) a.dsum[wrow + p0 + tid] = sD[tid];
    f32x16 x = mm_nt(tA, tB, z16(), wave, lane);            // X[i][m]
#pragma unroll
    for (int v = 0; v < 16; ++v)
        if (n > qrow(wave, lane, v)) x[v] = 0.f;            // lower: m <= i
    st_q<false>(tX, x, wave, lane);
    st_q<true>(tXT, x, wave, lane);
    __syncthreads();
    f32x16 s = mm_nt(tA, tC, z16(), wave, lane);            // Q K^T
    f32x16 xy = mm_nt(tX, tD, z16(), wave, lane);           // lower(X) Y
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
    // dS row sums accumulate per lane over every key chunk (one reduction
    // at the end); column sums of the own chunk's dS
    f32x16 rs = ds;
    {
        float cs = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) cs += ds[v];
        cs += __shfl_xor(cs, 32, 64);
        if (lane < 32) atomicAdd(&sCol[n], cs);
    }
    __syncthreads();                          // tile reads done
    st_q<false>(tB, ds, wave, lane);          // dS [i][j]
    st_q<true>(tC, ds, wave, lane);           // dS^T [j][i]
    st_q<true>(tD, pp, wave, lane);           // P^T [j][i]
    put_t(tE, fo, tid);                       // dO^T [d][i]
    put_t(tF, fq, tid);                       // Q^T [d][i]
    __syncthreads();
    // dV_own = P^T dO, dK_own = scale dS^T Q, dY = -scale lower(X)^T dS
    st_qg(own + 1 * BC * BC, mm_nt(tD, tE, z16(), wave, lane), wave, lane);
    st_qg(own + 0 * BC * BC, mm_nt(tC, tF, z16(), wave, lane), wave, lane, a.scale);
    st_qg(own + 2 * BC * BC, mm_nt(tXT, tC, z16(), wave, lane), wave, lane, -a.scale);
    __syncthreads();
    put_t(tD, fk, tid);                       // K^T [d][j]
    put(tE, fy, tid);                         // Y [m][j]
    put_t(tF, fu, tid);                       // U^T [e][m]
    __syncthreads();
    {
        const f32x16 dq = mm_nt(tB, tD, z16(), wave, lane);      // dS K, unscaled
        // dXl = -scale dS Y^T (lower)
        f32x16 dxl = mm_nt(tB, tE, z16(), wave, lane);
#pragma unroll
        for (int v = 0; v < 16; ++v) dxl[v] = (n <= qrow(wave, lane, v)) ? -a.scale * dxl[v] : 0.f;
        st_qg(own + 7 * BC * BC, dq, wave, lane, a.scale);
        st_qg(own + 8 * BC * BC, dxl, wave, lane);
    }

    // ---- Q~ = Q - lower(X) U (the query carried to the chunk start) ----
    f32x16 qc = mm_nt(tX, tF, z16(), wave, lane);           // lower(X) U
#pragma unroll
    for (int v = 0; v < 16; ++v) qc[v] = static_cast<float>(tA[qrow(wave, lane, v) * BP + n]) - qc[v];

    // ---- right to left: Q_{a,b}, b = a-1 .. 0, stored ----
    const size_t pairs = (size_t)N * (N - 1) / 2;
    bf16* qs = static_cast<bf16*>(a.qs) + (size_t)head * pairs * BC * BC;
    bf16* gs = static_cast<bf16*>(a.gs) + (size_t)head * pairs * BC * BC;
    // M_b and M_{b-1} in flight
    Frag fm = {}, fm1 = {};
    if (ca - 1 >= 1) fm = fetch(mn + (size_t)(ca - 1) * BC * BC, BC, tid);
    if (ca - 2 >= 1) fm1 = fetch(mn + (size_t)(ca - 2) * BC * BC, BC, tid);
    for (int b = ca - 1; b >= 0; --b) {
        __syncthreads();
        st_q<false>(tB, qc, wave, lane);                    // Q_{a,b}
        if (b >= 1) put_t(tC, fm, tid);                     // M_b^T [y][x]
        __syncthreads();
        fm = fm1;
        if (b - 2 >= 1) fm1 = fetch(mn + (size_t)(b - 2) * BC * BC, BC, tid);
        store_tile(qs + pair_index(ca, b) * BC * BC, tB, tid);
        if (b >= 1) {
            const f32x16 qm = mm_nt(tB, tC, z16(), wave, lane);   // Q M_b
#pragma unroll
            for (int v = 0; v < 16; ++v) qc[v] -= qm[v];
        }
    }
    // ---- left to right: dS_ab, the adjoint G, dQ_{a,b} ----
    double fsum = 0.0;                                       // sum of csum over chunks b+1 .. a (log2)
    if (gate)
        for (int c = 1; c <= ca; ++c) fsum += static_cast<double>(a.csum[chunk0 + c]);
    f32x16 g = z16();
    Frag fQ = {}, fK = {}, fV = {};
    float locK = 0.f;
    // csum of chunk b + 1, subtracted at the end of step b (loaded a step ahead)
    float cs_cur = (gate && ca >= 1) ? a.csum[chunk0 + 1] : 0.f, cs_nxt = 0.f;
    __syncthreads();                                         // Q_{a,b} stores visible
    if (ca >= 1) {
        fQ = fetch(qs + pair_index(ca, 0) * BC * BC, BC, tid);
        fK = fetch(ktw, BC, tid);
        fV = fetch(vv + hrow * BC, BC, tid);
        if (gate && tid < BC) locK = a.loc[wrow + tid];
    }
    put(tE, fetch(dO, nva, tid), tid);                       // dO [i][d]
    for (int b = 0; b < ca; ++b) {
        __syncthreads();
        put(tA, fQ, tid);                                    // Q_{a,b}
        put(tC, fK, tid);                                    // K~_b [j][d]
        put_t(tD, fK, tid);                                  // K~_b^T [d][j]
        put(tF, fV, tid);                                    // V_b (chunks left of a are full)
        if (b >= 1) put(tB, fm, tid);                        // M_b [x][y]
        st_q<false>(tX, g, wave, lane);                      // G_{b-1}
        if (tid < BC) sLocK[tid] = locK;
        __syncthreads();
        if (b + 1 < ca) {                                    // the next step's tiles
            fQ = fetch(qs + pair_index(ca, b + 1) * BC * BC, BC, tid);
            fK = fetch(ktw + (size_t)(b + 1) * BC * BC, BC, tid);
            fV = fetch(vv + (hrow + (size_t)(b + 1) * BC) * BC, BC, tid);
            fm = fetch(mn + (size_t)(b + 1) * BC * BC, BC, tid);
            if (gate && tid < BC) locK = a.loc[wrow + (size_t)(b + 1) * BC + tid];
        }
        if (gate && b + 2 <= ca) cs_nxt = a.csum[chunk0 + b + 2];
        if (b >= 1) store_tile(gs + pair_index(ca, b) * BC * BC, tX, tid);
        const float bias_q = static_cast<float>(fsum);
        const f32x16 sb = mm_nt(tA, tC, z16(), wave, lane);  // Q_{a,b} K~_b^T
        const f32x16 db = mm_nt(tE, tF, z16(), wave, lane);  // dO V_b^T
        f32x16 dsb;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int i = qrow(wave, lane, v);
            const float z = c2 * sb[v] + (gate ? sLoc[i] + bias_q - sLocK[n] : 0.f);
            const float p = i < nva ? exp2f(z - sLse[i]) : 0.f;
            dsb[v] = p * (db[v] - sD[i]);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) rs[v] += dsb[v];
        f32x16 gm = z16();
        if (b >= 1) gm = mm_nt(tX, tB, z16(), wave, lane);   // G_{b-1} M_b^T
        __syncthreads();                                     // tB, tX reads done
        st_q<false>(tB, dsb, wave, lane);                    // dS [i][j]
        __syncthreads();
        const f32x16 dqb = mm_nt(tB, tD, z16(), wave, lane); // dS K~_b
#pragma unroll
        for (int v = 0; v < 16; ++v) g[v] = a.scale * dqb[v] + (b >= 1 ? g[v] - gm[v] : 0.f);
        fsum -= static_cast<double>(cs_cur);
        cs_cur = cs_nxt;
    }
    // ---- dQ~ = G_{a-1}: Q~ backward.  dQ += dQ~ ; dXl += -(dQ~ U^T) lower ;
    // dU = -lower(X)^T dQ~ ; then dQ += dXl W, dW_own = dXl^T Q ----
    fu = fetch(un, BC, tid);
    fw = fetch(w, nva, tid);
    fq = fetch(q, nva, tid);
    __syncthreads();
    st_q<false>(tA, g, wave, lane);                          // dQ~ [i][e]
    st_q<true>(tB, g, wave, lane);                           // dQ~^T [e][i]
    put(tC, fu, tid);                                        // U [m][e]
    put_t(tD, fw, tid);                                      // W^T [d][m]
    put_t(tF, fq, tid);                                      // Q^T [d][i]
    __syncthreads();
    const f32x16 du = mm_nt(tA, tC, z16(), wave, lane);      // (dQ~ U^T)[i][m]
    f32x16 dq = ld_qg(own + 7 * BC * BC, wave, lane);
    f32x16 dxl = ld_qg(own + 8 * BC * BC, wave, lane);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        dq[v] += g[v];
        dxl[v] -= (n <= qrow(wave, lane, v)) ? du[v] : 0.f;
    }
    // dU = -lower(X)^T dQ~: rows m, cols e
    st_qg(own + 3 * BC * BC, mm_nt(tXT, tB, z16(), wave, lane), wave, lane, -1.f);
    __syncthreads();
    st_q<false>(tA, dxl, wave, lane);                        // dXl [i][m]
    st_q<true>(tB, dxl, wave, lane);                         // dXl^T [m][i]
    __syncthreads();
    const f32x16 dqw = mm_nt(tA, tD, z16(), wave, lane);     // dXl W
    st_qg(own + 4 * BC * BC, mm_nt(tB, tF, z16(), wave, lane), wave, lane);   // dW_own = dXl^T Q
    {
        float* dqg = a.dq + (hrow + p0) * BC;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int i = qrow(wave, lane, v);
            if (i < nva) dqg[(size_t)i * BC + n] = dq[v] + dqw[v];
        }
    }
    __syncthreads();
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const float r = wave_sum32(rs[v]);
        if ((lane & 31) == 0) atomicAdd(&sRow[qrow(wave, lane, v)], r);
    }
    __syncthreads();
    if (tid < BC) {
        a.rsum[wrow + p0 + tid] = sRow[tid];
        a.csd[wrow + p0 + tid] = sCol[tid];
    }
}

// ---------------------------------------------------------------------------
// Key-stationary: one workgroup per (head, key chunk b): dV, dK~ and dM
// summed over the query chunks a > b.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 2) void path_bwd_key_kernel(const BwdKArgs a) {
    __shared__ __attribute__((aligned(16))) bf16 tA[BT], tB[BT], tC[BT], tD[BT], tE[BT], tF[BT],
        tH[BT], tI[BT];
    __shared__ float sLse[BC], sD[BC], sLocQ[BC], sLocK[BC], sCol[BC];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int L = a.L, N = a.N, Lp = N * BC;
    int head, cb;
    wg_map(blockIdx.x, a.BH, N, false, head, cb);
    const int p0 = cb * BC, nvb = min(BC, L - p0);
    const size_t hrow = (size_t)head * L, wrow = (size_t)head * Lp;
    const size_t chunk0 = (size_t)head * N;
    const bool gate = a.loc != nullptr;
    const float c2 = a.scale * kLog2e;
    const int n = qcol(wave, lane);

    const bf16* vv = static_cast<const bf16*>(a.v);
    const bf16* dOg = static_cast<const bf16*>(a.dout);
    const bf16* ktw = static_cast<const bf16*>(a.kt) + wrow * BC;
    const size_t pairs = (size_t)N * (N - 1) / 2;
    const bf16* qs = static_cast<const bf16*>(a.qs) + (size_t)head * pairs * BC * BC;
    const bf16* gs = static_cast<const bf16*>(a.gs) + (size_t)head * pairs * BC * BC;
    float* own = a.own + (chunk0 + cb) * NOWN * BC * BC;

    // the tiles and per-query scalars of query chunk ca, in flight
    Frag fQ = {}, fO = {}, fG = {};
    float lse_n = 0.f, dsum_n = 0.f, loc_n = 0.f, cs_n = 0.f;
    auto prefetch = [&](int ca) {
        const int pa = ca * BC, nva = min(BC, L - pa);
        if (gate) cs_n = a.csum[chunk0 + ca];
        fQ = fetch(qs + pair_index(ca, cb) * BC * BC, BC, tid);
        fO = fetch(dOg + (hrow + pa) * BC, nva, tid);
        if (cb >= 1) fG = fetch(gs + pair_index(ca, cb) * BC * BC, BC, tid);
        if (tid < BC) {
            lse_n = tid < nva ? a.lse[hrow + pa + tid] * kLog2e : 0.f;
            dsum_n = a.dsum[wrow + pa + tid];
            loc_n = gate ? a.loc[wrow + pa + tid] : 0.f;
        }
    };
    if (cb + 1 < N) prefetch(cb + 1);
    {
        const Frag fk = fetch(ktw + (size_t)cb * BC * BC, BC, tid);
        const Frag fv = fetch(vv + (hrow + p0) * BC, nvb, tid);
        put(tA, fk, tid);                                            // K~_b [j][d]
        put(tB, fv, tid);                                            // V_b [j][d]
    }
    if (tid < BC) {
        sLocK[tid] = gate ? a.loc[wrow + p0 + tid] : 0.f;
        sCol[tid] = 0.f;
    }
    f32x16 dv = z16(), dkt = z16(), dm = z16();
    double fsum = 0.0;     // sum of csum over chunks b+1 .. a
    for (int ca = cb + 1; ca < N; ++ca) {
        const int nva = min(BC, L - ca * BC);
        fsum += static_cast<double>(cs_n);
        __syncthreads();
        put(tC, fQ, tid);                                            // Q_{a,b} [i][d]
        put_t(tD, fQ, tid);                                          // Q_{a,b}^T [d][i]
        put(tE, fO, tid);                                            // dO_a [i][d]
        put_t(tF, fO, tid);                                          // dO_a^T [d][i]
        if (cb >= 1) put_t(tH, fG, tid);                             // G^T [y][i]
        if (tid < BC) {
            sLse[tid] = lse_n;
            sD[tid] = dsum_n;
            sLocQ[tid] = loc_n;
        }
        __syncthreads();
        if (ca + 1 < N) prefetch(ca + 1);
        const float bias_q = static_cast<float>(fsum);
        const f32x16 sb = mm_nt(tC, tA, z16(), wave, lane);         // Q K~^T [i][j]
        const f32x16 db = mm_nt(tE, tB, z16(), wave, lane);         // dO V^T [i][j]
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
    // dV = P^T dO (later queries) + own chunk; dK~ and dM for the UT kernel
    {
        const f32x16 dvo = ld_qg(own + 1 * BC * BC, wave, lane);
        float* dvg = a.dv + (hrow + p0) * BC;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int j = qrow(wave, lane, v);
            if (j < nvb) dvg[(size_t)j * BC + n] = dv[v] + dvo[v];
        }
    }
    st_qg(own + 5 * BC * BC, dkt, wave, lane, a.scale);
    st_qg(own + 6 * BC * BC, dm, wave, lane, -1.f);
    __syncthreads();
    if (tid < BC) a.csl[wrow + p0 + tid] = sCol[tid];
}

// ---------------------------------------------------------------------------
// UT-transform backward of one chunk.  Inputs: dK~, dM (key kernel) and
// dU, dY, the own-chunk dK, dW (query kernel).  Recomputed: G = W W^T,
// X = (I + A)^{-1} with A = strictLower(D G), T^{-1} = X D,
// R = strictLower(W K^T), Y = T^{-1} R, U = T^{-1} W.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void path_bwd_ut_kernel(const BwdKArgs a) {
    __shared__ __attribute__((aligned(16))) bf16 tA[BT], tB[BT], tCt[BT], tD[BT], tE[BT],
        tF[BT], tH[BT], tI[BT];
    __shared__ __attribute__((aligned(16))) float sG[BC * FP], sX[BC * FP];   // fp32: G, (I + A)^{-1}
    __shared__ float sB[BC], sDb[BC];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int L = a.L, N = a.N;
    const int head = blockIdx.x / N, cb = blockIdx.x % N;
    const int p0 = cb * BC, nvb = min(BC, L - p0);
    const size_t hrow = (size_t)head * L;
    const int n = qcol(wave, lane);
    const float* own = a.own + ((size_t)head * N + cb) * NOWN * BC * BC;

    // Tiles: tA W [m][e], tB W^T [e][m], tCt K [j][e], tD K^T [e][j],
    // tE T^{-1} [m][n], tF T^{-1}^T [n][m]; tH, tI scratch.
    {
        const Frag fw = fetch(static_cast<const bf16*>(a.w) + (hrow + p0) * BC, nvb, tid);
        const Frag fk = fetch(static_cast<const bf16*>(a.k) + (hrow + p0) * BC, nvb, tid);
        put(tA, fw, tid);
        put_t(tB, fw, tid);
        put(tCt, fk, tid);
        put_t(tD, fk, tid);
    }
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
    // X = (I + A)^{-1} (unit lower triangular) by forward substitution on
    // wave 0, lane c holding column c in registers:
    // X[m][c] = delta_mc - beta_m sum_{p < m} G[m][p] X[p][c], where X[p][c] = 0
    // for p < c makes every m <= c give delta_mc.
    if (wave == 0) {
        float t[BC];
#pragma unroll
        for (int m = 0; m < BC; ++m) {
            const float* grow = sG + m * FP;
            float acc = 0.f;
#pragma unroll
            for (int p = 0; p < m; ++p) acc = fmaf(grow[p], t[p], acc);
            t[m] = (m == lane ? 1.f : 0.f) - sB[m] * acc;
        }
#pragma unroll
        for (int m = 0; m < BC; ++m) sX[m * FP + lane] = t[m];
    }
    __syncthreads();
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
    const f32x16 dkt = ld_qg(own + 5 * BC * BC, wave, lane);        // dK~
    const f32x16 dm = ld_qg(own + 6 * BC * BC, wave, lane);         // dM
#pragma unroll
    for (int v = 0; v < 16; ++v) dK[v] += dkt[v];                    // K~ = K - Y^T W
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
        const bf16 xv = static_cast<bf16>(sX[m * FP + c]);
        tI[m * BP + c] = xv;                                         // X [p][c]
        tCt[c * BP + m] = xv;                                        // X^T [c][m]
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
    // inclusive suffix sums of the run totals
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
    hipLaunchKernelGGL(path_bwd_layout_kernel, grid, block, 0, s, a);
    hipLaunchKernelGGL(path_bwd_query_kernel, grid, block, 0, s, a);
    hipLaunchKernelGGL(path_bwd_key_kernel, grid, block, 0, s, a);
    hipLaunchKernelGGL(path_bwd_ut_kernel, grid, block, 0, s, a);
    if (a.log_f) hipLaunchKernelGGL(path_bwd_gate_kernel, dim3(a.BH), block, 0, s, a);
    return hipGetLastError();
}

}  // namespace path
