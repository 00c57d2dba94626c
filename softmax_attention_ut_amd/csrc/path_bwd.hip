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
// and the gate sums), each a grid over (head, chunk):
//   path_bwd_layout_kernel   U, Y as row-major tiles (in place) and the
//       operand tiles of the chains (K~, scale K~^T, -M, -M^T with the k
//       axis in the accumulator slot order, see below);
//   path_bwd_own_kernel      a query chunk's own-chunk step (probabilities,
//       dV, dK, dY of the chunk itself, the partial dQ and d lower(Q W^T))
//       and Q~, the query carried to the chunk start;
//   path_bwd_chain_kernel    two query chunks per workgroup: Q_{a,b} right
//       to left (stored per pair), then the adjoint G left to right (stored
//       per pair) -> dQ~ = G_{a-1} and the row sums of dS;
//   path_bwd_own_end_kernel  dQ~ through Q~ = Q - lower(Q W^T) U: dQ, dU, dW
//       of the own chunk;
//   path_bwd_key_kernel      one key chunk per workgroup: dV, dK~, dM summed
//       over the later query chunks, and the column sums of dS;
//   path_bwd_ut_kernel       the UT-transform backward -> dK, dW, dbeta;
//   path_bwd_gate_kernel     dlog f by suffix sums.
// The own-chunk kernels work on 64 x 64 LDS tiles with four waves, each wave
// a 32 x 32 quarter of every product.  The chain and key kernels keep their
// states in MFMA accumulators: in the 32x32x16 bf16 MFMA, accumulator
// registers 8s .. 8s+7 of a 32 x 32 tile are exactly the B operand of k-step
// s when the k axis is taken in the slot order permk (path_internal.h), so a
// product's result feeds the next product with no data movement, and every
// A operand that meets it is stored with its k axis in that order.  The
// per-pair states (Q_{a,b}, G_{a,b-1}) are stored as bf16 rows in slot
// order, which is both the chain kernel's B operand and the key kernel's A
// operand.
#include "path_internal.h"

namespace path {

namespace {

constexpr int BC = 64;        // chunk = head dim
constexpr int BP = BC + 8;    // LDS tile pitch (bf16 elements)
constexpr int BT = BC * BP;   // LDS tile size (elements)
constexpr int FP = BC + 4;    // fp32 LDS tile pitch (rows 16-byte aligned)
constexpr int TT = BC * BC;   // elements of a 64 x 64 workspace tile
constexpr int NOWN = 11;      // fp32 64 x 64 partials per chunk (see below)

__device__ __forceinline__ f32x16 mfmab(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 l8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ void s8(bf16* p, bf16x8 x) { *reinterpret_cast<bf16x8*>(p) = x; }
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
// quarter -> two bf16 LDS tiles, x * s = hi + lo to about 16 bits
// (hi = bf16(x * s), lo = bf16(x * s - hi)), as is or transposed
template <bool TR>
__device__ __forceinline__ void st_q2(bf16* Th, bf16* Tl, const f32x16& acc, int wave, int lane,
                                      float s = 1.f) {
    const int n = qcol(wave, lane);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int m = qrow(wave, lane, v);
        const float x = s * acc[v];
        const bf16 h = static_cast<bf16>(x);
        const bf16 l = static_cast<bf16>(x - static_cast<float>(h));
        const int o = TR ? n * BP + m : m * BP + n;
        Th[o] = h;
        Tl[o] = l;
    }
}
// acc += (Ah + Al)(Bh + Bl)^T without the lo x lo term: three bf16 products
__device__ __forceinline__ f32x16 mm_nt3(const bf16* Ah, const bf16* Al, const bf16* Bh,
                                         const bf16* Bl, f32x16 acc, int wave, int lane) {
    acc = mm_nt(Ah, Bh, acc, wave, lane);
    acc = mm_nt(Ah, Bl, acc, wave, lane);
    return mm_nt(Al, Bh, acc, wave, lane);
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

// A 64 x 64 bf16 tile of row-major [64][64] global rows in flight over 256
// threads: thread t holds rows 2 (t & 31) and 2 (t & 31) + 1, columns
// 8 (t >> 5) .. + 7.  fetch issues the loads (rows >= nvalid read as zero);
// put / put_t write the fragment to an LDS tile as is or transposed (then
// each pair of rows is one 4-byte word per column: the 64 lanes of a wave
// hit 64 distinct banks).
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
    s8(T + r * BP + c, f.x[0]);
    s8(T + (r + 1) * BP + c, f.x[1]);
}
__device__ __forceinline__ void put_t(bf16* T, const Frag& f, int tid) {
    const int r = 2 * (tid & 31), c = 8 * (tid >> 5);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const bf16x2 p = {f.x[0][e], f.x[1][e]};
        *reinterpret_cast<bf16x2*>(T + (c + e) * BP + r) = p;
    }
}
// Transposed with the old row index taken into slot order: T[col][permk(row)]
// (a tile whose rows become the k axis of a chained product); put_tp also
// takes the old column into slot order: T[permk(col)][permk(row)].  permk
// keeps the rows 2i, 2i+1 adjacent.
__device__ __forceinline__ void put_to(bf16* T, const Frag& f, int tid) {
    const int r = 2 * (tid & 31), c = 8 * (tid >> 5), pr = permk(r);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const bf16x2 p = {f.x[0][e], f.x[1][e]};
        *reinterpret_cast<bf16x2*>(T + (c + e) * BP + pr) = p;
    }
}
__device__ __forceinline__ void put_tp(bf16* T, const Frag& f, int tid) {
    const int r = 2 * (tid & 31), c = 8 * (tid >> 5), pr = permk(r);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const bf16x2 p = {f.x[0][e], f.x[1][e]};
        *reinterpret_cast<bf16x2*>(T + permk(c + e) * BP + pr) = p;
    }
}
// LDS tile -> row-major [64][64] global rows (16-byte stores)
__device__ __forceinline__ void store_tile(bf16* g, const bf16* T, int tid) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int u = tid + 256 * it, r = u >> 3, c = (u & 7) * 8;
        s8(g + r * BC + c, l8(T + r * BP + c));
    }
}

// Accumulator registers 8 H .. 8 H + 7 as a bf16 B operand (times s).
template <int H>
__device__ __forceinline__ bf16x8 cvt8(const f32x16& a, float s = 1.f) {
    bf16x8 r;
#pragma unroll
    for (int t = 0; t < 8; ++t) r[t] = static_cast<bf16>(s * a[8 * H + t]);
    return r;
}
// B operand of k-step ks from a pair of accumulator tiles (rows 0-31, 32-63)
__device__ __forceinline__ bf16x8 bop(const f32x16* acc, int ks, float s = 1.f) {
    return (ks & 1) ? cvt8<1>(acc[ks >> 1], s) : cvt8<0>(acc[ks >> 1], s);
}
// A operand of block blk (rows 32 blk ..), k-step ks from an LDS tile
__device__ __forceinline__ bf16x8 aop(const bf16* T, int blk, int ks, int lane) {
    return l8(T + (32 * blk + (lane & 31)) * BP + 16 * ks + 8 * (lane >> 5));
}
// acc[blk] += A(T) B over the 64-long k axis, for both row blocks
__device__ __forceinline__ void mm2(f32x16* acc, const bf16* T, const bf16x8* b, int lane) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a0 = aop(T, 0, ks, lane), a1 = aop(T, 1, ks, lane);
        acc[0] = mfmab(a0, b[ks], acc[0]);
        acc[1] = mfmab(a1, b[ks], acc[1]);
    }
}

// Swizzled unpadded tiles for the chain kernel's direct global -> LDS
// copies: 64 rows of 128 bytes, the 16-byte unit u of row r stored at unit
// u ^ swz(r), so that the 32 rows one A-operand read touches fall on
// distinct banks.
__device__ __forceinline__ int swz(int r) { return (r ^ ((r >> 3) & 3)) & 7; }
__device__ __forceinline__ bf16x8 aop_s(const bf16* T, int blk, int ks, int lane) {
    const int r = 32 * blk + (lane & 31);
    return l8(T + r * BC + 8 * ((2 * ks + (lane >> 5)) ^ swz(r)));
}
__device__ __forceinline__ void mm2_s(f32x16* acc, const bf16* T, const bf16x8* b, int lane) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a0 = aop_s(T, 0, ks, lane), a1 = aop_s(T, 1, ks, lane);
        acc[0] = mfmab(a0, b[ks], acc[0]);
        acc[1] = mfmab(a1, b[ks], acc[1]);
    }
}
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ unsigned lds_addr(const void* p) {
    return static_cast<unsigned>(reinterpret_cast<uintptr_t>((const lds_void*)p));
}
// global -> LDS copy of 16 (or 4) bytes per lane: lane i writes lds + 16 i
// (4 i) from gbase + voff.  Issued as inline assembly, out of the
// compiler's sight (it would otherwise wait for such copies at its own
// points, with all older stores): the caller waits with s_waitcnt vmcnt.
// The copy takes its LDS base from M0, which is saved and restored around it.
__device__ __forceinline__ void dma16(const void* gbase, unsigned voff, const void* lds) {
    unsigned keep;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
                 : "=&s"(keep) : "v"(voff), "s"(gbase), "s"(lds_addr(lds)) : "memory");
}
__device__ __forceinline__ void dma4(const void* gbase, unsigned voff, const void* lds) {
    unsigned keep;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
                 "global_load_lds_dword %1, %2\n\ts_mov_b32 m0, %0"
                 : "=&s"(keep) : "v"(voff), "s"(gbase), "s"(lds_addr(lds)) : "memory");
}
// Wait until at most n vector memory operations of this wave are in flight
// (they complete in issue order): n = the stores issued after the copies
// being waited for.
__device__ __forceinline__ void wait_vm(int n) {
    switch (n) {
        case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
        case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
        case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
        case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
        case 16: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
}

// Workgroup barrier without the memory fence of __syncthreads (which waits
// for every store of the wave to complete): the chain kernel's LDS tiles come
// from the copies above, each wave having waited for its own.
__device__ __forceinline__ void bar() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The probabilities are v_exp_f32 of their log2 argument (no range
// reduction: results below the smallest normal flush to zero, which is far
// below the bf16 rounding of any probability that counts).

__device__ __forceinline__ float wave_sum32(float x) {   // over the 32 lanes of a half
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) x += __shfl_xor(x, off, 32);
    return x;
}

// Workgroup -> (head, unit).  Workgroups are dealt to the 8 XCDs in turn;
// when B*H is a multiple of 8, head h goes to XCD h % 8 and its units run
// together there, so the per-chunk tiles every unit of a head reads stay in
// that XCD's L2.  rev: units in decreasing order.
__device__ __forceinline__ void wg_map(int x, int BH, int NU, bool rev, int& head, int& u) {
    if ((BH & 7) == 0) {
        const int slot = x >> 3;
        head = (slot / NU) * 8 + (x & 7);
        u = slot % NU;
    } else {
        head = x / NU;
        u = x % NU;
    }
    if (rev) u = NU - 1 - u;
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
//   qs, gs   [BH][pairs][64][64] bf16  Q_{a,b} and G_{a,b-1} (b >= 1), rows
//                                      i with the d axis in slot order:
//                                      qs[i][s] = Q_{a,b}[i][permk(s)]
//   kp, kts, mn, mtn [BH][N][64][64] bf16, per chunk (slot order s):
//            kp[j][s] = K~[j][permk(s)]          kts[e][s] = scale K~[permk(s)][e]
//            mn[x][s] = -M[x][permk(s)]          mtn[y][s] = -M[permk(s)][y]
//   own      [BH][N][11][64][64] fp32  per chunk: dK (own-chunk step), dV
//                                      (own chunk), dY, dU, dW (own chunk),
//                                      dK~, dM, the own-chunk dQ and
//                                      d lower(Q W^T), Q~ and dQ~
//   dsum     [BH][Lp] fp32   rowsum(dO o O) per query
//   rsum     [BH][Lp] fp32   rowsum(dS) per query (all its keys)
//   csd      [BH][Lp] fp32   colsum(dS) of the own-chunk step per key
//   csl      [BH][Lp] fp32   colsum(dS) over the later query chunks per key
// ut, yt hold U, Y as row-major tiles once path_bwd_layout_kernel ran.
using BwdKArgs = BwdArgs;

// ---------------------------------------------------------------------------
// Per chunk: U, Y from the prepare stage's operand layouts to row-major
// tiles, in place, and the chains' operand tiles.  The prepare stage's
// layouts (permk = its k-slot permutation):
//   ut[rho][sigma] = -U[permk(sigma)][permk(rho)]   -> U[m][e]
//   yt[j][sigma]   =  Y[permk(sigma)][j]            -> Y[m][j]
//   mt[rho][e]     = -M[e][permk(rho)], so -M[x][permk(s)] = mt[s][x] and
//                    -M[permk(s)][y] = mt[permk(y)][permk(s)]
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void path_bwd_layout_kernel(const BwdKArgs a) {
    __shared__ __attribute__((aligned(16))) bf16 tU[BT], tY[BT], tM[BT], tK[BT];
    const int tid = threadIdx.x;
    const size_t base = (size_t)blockIdx.x * TT;
    bf16* ut = static_cast<bf16*>(a.ut) + base;
    bf16* yt = static_cast<bf16*>(a.yt) + base;
    const bf16* mt = static_cast<const bf16*>(a.mt) + base;
    const Frag fk = fetch(static_cast<const bf16*>(a.kt) + base, BC, tid);   // K~ rows
    bf16 xu[16], xy[16];
#pragma unroll
    for (int it = 0; it < 16; ++it) {
        const int u = tid + 256 * it;
        xu[it] = ut[u];
        xy[it] = yt[u];
    }
    const Frag fm = fetch(mt, BC, tid);
#pragma unroll
    for (int it = 0; it < 16; ++it) {
        const int u = tid + 256 * it, hi = u >> 6, lo = u & 63;
        tU[permk(lo) * BP + permk(hi)] = static_cast<bf16>(-static_cast<float>(xu[it]));
        tY[permk(lo) * BP + hi] = xy[it];
    }
    put(tM, fm, tid);          // mt as is
    put(tK, fk, tid);          // K~ as is
    __syncthreads();
    store_tile(ut, tU, tid);
    store_tile(yt, tY, tid);
    bf16* kp = static_cast<bf16*>(a.kp) + base;
    bf16* kts = static_cast<bf16*>(a.kts) + base;
    bf16* mn = static_cast<bf16*>(a.mn) + base;
    bf16* mtn = static_cast<bf16*>(a.mtn) + base;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int u = tid + 256 * it, r = u >> 3, s0 = (u & 7) * 8;
        bf16x8 vkp, vkt, vmn, vmt;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int s = s0 + t, ps = permk(s);
            vkp[t] = tK[r * BP + ps];
            vkt[t] = static_cast<bf16>(a.scale * static_cast<float>(tK[ps * BP + r]));
            vmn[t] = tM[s * BP + r];
            vmt[t] = tM[permk(r) * BP + ps];
        }
        s8(kp + r * BC + s0, vkp);
        s8(kts + r * BC + s0, vkt);
        s8(mn + r * BC + s0, vmn);
        s8(mtn + r * BC + s0, vmt);
    }
}

// ---------------------------------------------------------------------------
// Own chunk of query chunk a (four waves, 64 x 64 LDS tiles): the chunk's
// probabilities from S_aa, its dV, dK, dY contributions, the partial dQ and
// d lower(Q W^T), rowsum(dO o O), the own row and column sums of dS, and Q~.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 2) void path_bwd_own_kernel(const BwdKArgs a) {
    __shared__ __attribute__((aligned(16))) bf16 tA[BT], tB[BT], tC[BT], tD[BT], tE[BT], tF[BT],
        tX[BT], tXT[BT];
    __shared__ float sLse[BC], sD[BC], sLoc[BC], sRow[BC], sCol[BC];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int L = a.L, N = a.N, Lp = N * BC;
    int head, ca;
    wg_map(blockIdx.x, a.BH, N, false, head, ca);
    const int p0 = ca * BC, nva = min(BC, L - p0);
    const size_t hrow = (size_t)head * L;      // input rows of the head
    const size_t wrow = (size_t)head * Lp;     // workspace rows of the head
    const size_t chunk0 = (size_t)head * N;    // first chunk of the head
    const bool gate = a.loc != nullptr;
    const float c2 = a.scale * kLog2e;
    const int n = qcol(wave, lane);

    const bf16* q = static_cast<const bf16*>(a.q) + (hrow + p0) * BC;
    const bf16* k = static_cast<const bf16*>(a.k) + (hrow + p0) * BC;
    const bf16* vv = static_cast<const bf16*>(a.v) + (hrow + p0) * BC;
    const bf16* w = static_cast<const bf16*>(a.w) + (hrow + p0) * BC;
    const bf16* o = static_cast<const bf16*>(a.out) + (hrow + p0) * BC;
    const bf16* dO = static_cast<const bf16*>(a.dout) + (hrow + p0) * BC;
    const bf16* un = static_cast<const bf16*>(a.ut) + (chunk0 + ca) * TT;
    const bf16* yn = static_cast<const bf16*>(a.yt) + (chunk0 + ca) * TT;
    float* own = a.own + (chunk0 + ca) * NOWN * TT;

    // S = scale (Q K^T - lower(X) Y) + gate, X = Q W^T
    const Frag fq = fetch(q, nva, tid), fw = fetch(w, nva, tid), fk = fetch(k, nva, tid);
    const Frag fy = fetch(yn, BC, tid), fo = fetch(dO, nva, tid);
    const Frag fv = fetch(vv, nva, tid), fu = fetch(un, BC, tid);
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
    f32x16 ds, pp;
    {
        const f32x16 s = mm_nt(tA, tC, z16(), wave, lane);      // Q K^T
        const f32x16 xy = mm_nt(tX, tD, z16(), wave, lane);     // lower(X) Y
        const f32x16 dp = mm_nt(tE, tF, z16(), wave, lane);     // dO V^T
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int i = qrow(wave, lane, v);
            const float z = c2 * (s[v] - xy[v]) + (sLoc[i] - sLoc[n]);
            const float p = (n <= i && i < nva) ? __builtin_amdgcn_exp2f(z - sLse[i]) : 0.f;
            pp[v] = p;
            ds[v] = p * (dp[v] - sD[i]);
        }
    }
    // row and column sums of the own chunk's dS
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
    __syncthreads();                          // tile reads done
    st_q<false>(tB, ds, wave, lane);          // dS [i][j]
    st_q<true>(tC, ds, wave, lane);           // dS^T [j][i]
    st_q<true>(tD, pp, wave, lane);           // P^T [j][i]
    put_t(tE, fo, tid);                       // dO^T [d][i]
    put_t(tF, fq, tid);                       // Q^T [d][i]
    __syncthreads();
    // dV_own = P^T dO, dK_own = scale dS^T Q, dY = -scale lower(X)^T dS
    st_qg(own + 1 * TT, mm_nt(tD, tE, z16(), wave, lane), wave, lane);
    st_qg(own + 0 * TT, mm_nt(tC, tF, z16(), wave, lane), wave, lane, a.scale);
    st_qg(own + 2 * TT, mm_nt(tXT, tC, z16(), wave, lane), wave, lane, -a.scale);
    __syncthreads();
    put_t(tD, fk, tid);                       // K^T [d][j]
    put(tE, fy, tid);                         // Y [m][j]
    put_t(tF, fu, tid);                       // U^T [e][m]
    __syncthreads();
    {
        // dQ (own chunk) = scale dS K; dXl = -scale dS Y^T (lower)
        const f32x16 dq = mm_nt(tB, tD, z16(), wave, lane);
        f32x16 dxl = mm_nt(tB, tE, z16(), wave, lane);
#pragma unroll
        for (int v = 0; v < 16; ++v) dxl[v] = (n <= qrow(wave, lane, v)) ? -a.scale * dxl[v] : 0.f;
        st_qg(own + 7 * TT, dq, wave, lane, a.scale);
        st_qg(own + 8 * TT, dxl, wave, lane);
    }
    {
        // Q~ = Q - lower(X) U, the query carried to the chunk start (fp32)
        f32x16 qc = mm_nt(tX, tF, z16(), wave, lane);
#pragma unroll
        for (int v = 0; v < 16; ++v) qc[v] = static_cast<float>(tA[qrow(wave, lane, v) * BP + n]) - qc[v];
        st_qg(own + 9 * TT, qc, wave, lane);
    }
    if (tid < BC) {
        a.rsum[wrow + p0 + tid] = sRow[tid];
        a.csd[wrow + p0 + tid] = sCol[tid];
    }
}

// ---------------------------------------------------------------------------
// The chains of two query chunks of a head (waves 0, 1: chunk a_hi = N-1-2p,
// queries 0-31 and 32-63; waves 2, 3: chunk a_hi - 1), which share the
// per-key-chunk operand tiles.  Each wave holds its 32 queries as columns of
// 64 x 32 accumulator pairs (rows = the d or key axis).
//   right to left:  Q^T <- Q^T + (-M_b^T) Q^T,   storing Q_{a,b}, b = a-1 .. 0;
//   left to right:  S^T = K~_b Q^T, dP^T = V_b dO^T, dS^T,
//                   G^T <- G^T + (-M_b) G^T + (scale K~_b^T) dS^T,
//                   storing G_{a,b-1} (b >= 1); dQ~ = G_{a-1}.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 2) void path_bwd_chain_kernel(const BwdKArgs a) {
    // Eight swizzled [64][64] tiles in two sets of four: the right-to-left
    // pass stages blocks of four -M_b^T tiles, the left-to-right pass a step's
    // K~_b, scale K~_b^T, V_b, -M_b; one set is read while the other fills.
    __shared__ __attribute__((aligned(1024))) bf16 tb[8 * TT];
    // sLoc[s][0..63]: the key chunk's gate terms; sLoc[s][64]: csum of chunk b + 1
    __shared__ __attribute__((aligned(16))) float sLoc[2][BC + 4];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int L = a.L, N = a.N, Lp = N * BC, NP = N / 2;
    int head, pr;
    wg_map(blockIdx.x, a.BH, NP, false, head, pr);
    const int ahi = N - 1 - 2 * pr;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int ca = ahi - (wave_u >> 1);            // this wave's query chunk (wave-uniform)
    const bool has = ca >= 1;                      // chunk 0 has no chain
    const int i = 32 * (wave & 1) + l32;           // the lane's query within the chunk
    const int row = ca * BC + i;
    const bool valid = row < L;
    const size_t hrow = (size_t)head * L, wrow = (size_t)head * Lp, chunk0 = (size_t)head * N;
    const bool gate = a.loc != nullptr;
    const float c2 = a.scale * kLog2e;
    const size_t pairs = (size_t)N * (N - 1) / 2;
    bf16* qs = static_cast<bf16*>(a.qs) + (size_t)head * pairs * TT;
    bf16* gs = static_cast<bf16*>(a.gs) + (size_t)head * pairs * TT;
    const bf16* kp = static_cast<const bf16*>(a.kp) + chunk0 * TT;
    const bf16* kts = static_cast<const bf16*>(a.kts) + chunk0 * TT;
    const bf16* mn = static_cast<const bf16*>(a.mn) + chunk0 * TT;
    const bf16* mtn = static_cast<const bf16*>(a.mtn) + chunk0 * TT;
    const bf16* vv = static_cast<const bf16*>(a.v) + hrow * BC;
    float* own = a.own + (chunk0 + ca) * NOWN * TT;

    // The per-query values of the left-to-right pass, loaded here with the
    // first right-to-left operands (one round trip for all of them).  fsum,
    // the sum of the chunk sums csum over chunks 1 .. a, is summed across the
    // wave (lane l takes chunks 1 + l, 65 + l, ...), not one load at a time.
    const float lse2 = (has && valid) ? a.lse[hrow + row] * kLog2e : 0.f;
    const float Di = has ? a.dsum[wrow + row] : 0.f;
    const float locQ = (gate && has) ? a.loc[wrow + row] : 0.f;
    bf16x8 dob[4];                                        // dO^T as the B operand (d natural)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        dob[ks] = bf16x8{};
        if (has && valid) dob[ks] = l8(static_cast<const bf16*>(a.dout) + (hrow + row) * BC + 16 * ks + 8 * hh);
    }
    double fsum = 0.0;                                    // sum of csum over chunks b+1 .. a (log2)
    if (gate && has) {
        for (int c = 1 + lane; c <= ca; c += 64) fsum += static_cast<double>(a.csum[chunk0 + c]);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) fsum += __shfl_xor(fsum, off, 64);
    }

    // This lane's part of a tile copy: 16-byte unit P = 256 j + 64 wave + lane
    // of the swizzled LDS tile (j = 0, 1) comes from row P / 8, logical unit
    // (P % 8) ^ swz(row) of the row-major global tile.
    unsigned goff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int P = 256 * j + 64 * wave + lane, r = P >> 3;
        goff[j] = static_cast<unsigned>(r * 128 + 16 * ((P & 7) ^ swz(r)));
    }
    auto copy_tile = [&](bf16* T, const bf16* g) {
#pragma unroll
        for (int j = 0; j < 2; ++j) dma16(g, goff[j], T + (256 * j + 64 * wave_u) * 8);
    };

    // ---- right to left ----
    f32x16 q[2];
    // blocks of four steps: block i (b = b0 .. b0 - 3, b0 = ahi - 1 - 4 i)
    // reads set i % 2; its -M_b^T tiles were copied during the block before
    auto copy_block = [&](int b0, int set) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
            if (b0 - t >= 1) copy_tile(tb + (4 * set + t) * TT, mtn + (size_t)(b0 - t) * TT);
    };
    copy_block(ahi - 1, 0);
    {
        // Q~ (fp32 rows) into the accumulator layout: register v of tile blk
        // holds d = 32 blk + 8 (v >> 2) + 4 hh + (v & 3)
        const float* qf = own + 9 * TT + i * BC;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                f32x4 x4 = {0.f, 0.f, 0.f, 0.f};
                if (has) x4 = *reinterpret_cast<const f32x4*>(qf + 32 * blk + 8 * g4 + 4 * hh);
#pragma unroll
                for (int r = 0; r < 4; ++r) q[blk][4 * g4 + r] = x4[r];
            }
    }
    {
        int stores = -1;                  // stores issued after the last copies (-1: wait for all)
        int set = 0;
        for (int b0 = ahi - 1; b0 >= 0; b0 -= 4, set ^= 1) {
            wait_vm(stores < 0 ? -1 : 4 * stores);
            bar();
            if (b0 - 4 >= 1) copy_block(b0 - 4, set ^ 1);
            stores = 0;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int b = b0 - t;
                if (b < 0) break;
                const bool mine = has && b <= ca - 1;
                bf16x8 qb[4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) qb[ks] = bop(q, ks);
                if (mine) {
                    bf16* dst = qs + pair_index(ca, b) * TT + i * BC + 8 * hh;
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) s8(dst + 16 * ks, qb[ks]);
                    ++stores;
                    if (b >= 1) mm2_s(q, tb + (4 * set + t) * TT, qb, lane);   // Q^T += (-M_b^T) Q^T
                }
            }
        }
    }

    // ---- left to right ----
    f32x16 g[2] = {z16(), z16()};
    float rs = 0.f;
    // step b reads set b % 2: K~_b (d in slot order), scale K~_b^T (keys in
    // slot order), V_b (chunks left of a are full), -M_b (k in slot order),
    // the gate terms; the next step's copies and queries are issued at its
    // start.
    auto copy_step = [&](int b, int set) {
        bf16* T = tb + 4 * set * TT;
        copy_tile(T, kp + (size_t)b * TT);
        copy_tile(T + TT, kts + (size_t)b * TT);
        copy_tile(T + 2 * TT, vv + (size_t)b * TT);
        copy_tile(T + 3 * TT, mn + (size_t)b * TT);
        if (gate && wave_u == 0) {
            dma4(a.loc + wrow + (size_t)b * BC, lane * 4, sLoc[set]);
            if (lane == 0) dma4(a.csum + chunk0 + b + 1, 0, sLoc[set] + BC);
        }
    };
    bf16x8 qn[4] = {};
    auto load_q = [&](int b) {
        if (has && b <= ca - 1) {
            const bf16* src = qs + pair_index(ca, b) * TT + i * BC + 8 * hh;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) qn[ks] = l8(src + 16 * ks);
        }
    };
    bar();                      // the last right-to-left block's tiles are read
    if (ahi >= 1) {
        copy_step(0, 0);
        load_q(0);
    }
    int stored = -1;                      // G stores issued after the last copies (-1: wait for all)
    for (int b = 0; b < ahi; ++b) {
        const int set = b & 1;
        const bool mine = has && b <= ca - 1;
        wait_vm(stored < 0 ? -1 : 4 * stored);
        bar();
        bf16x8 qc[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qc[ks] = qn[ks];
        if (b + 1 < ahi) {                                // the next step's operands
            copy_step(b + 1, set ^ 1);
            load_q(b + 1);
        }
        const bf16* tK = tb + 4 * set * TT;
        const float* lk = sLoc[set];
        // G_{a,b-1}, stored by every wave at every step (four stores each, so
        // that the waits above and the compiler's own waits for the queries
        // can count them): steps without such a state write to the slot of
        // the pair (a, 0), which nothing reads.
        bf16x8 gb[4];
        {
            const size_t slot = (mine && b >= 1) ? pair_index(ca, b) : pair_index(ca > 0 ? ca : 1, 0);
            bf16* dst = gs + slot * TT + i * BC + 8 * hh;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                gb[ks] = bop(g, ks);
                s8(dst + 16 * ks, gb[ks]);
            }
        }
        stored = 1;
        if (mine) {
            f32x16 s[2] = {z16(), z16()}, dp[2] = {z16(), z16()};
            mm2_s(s, tK, qc, lane);                        // S^T[j][i], unscaled
            mm2_s(dp, tK + 2 * TT, dob, lane);             // dP^T[j][i]
            // row offset of query i: the gate's local term and chunk sums, -lse
            const float rq = valid ? (locQ + static_cast<float>(fsum) - lse2) : -INFINITY;
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const f32x4 l4 = gate ? *reinterpret_cast<const f32x4*>(lk + 32 * blk + 8 * g4 + 4 * hh)
                                          : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int v = 4 * g4 + r;
                        const float p = __builtin_amdgcn_exp2f(c2 * s[blk][v] + rq - l4[r]);
                        const float d = p * (dp[blk][v] - Di);
                        rs += d;
                        s[blk][v] = d;                     // dS^T
                    }
                }
            bf16x8 db[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) db[ks] = bop(s, ks);
            if (b >= 1) mm2_s(g, tK + 3 * TT, gb, lane);   // G^T - M_b G^T
            mm2_s(g, tK + TT, db, lane);                   // + scale K~_b^T dS^T
        }
        if (gate) fsum -= static_cast<double>(lk[BC]);
    }
    if (has) {
        rs += __shfl_xor(rs, 32, 64);
        if (hh == 0 && valid) a.rsum[wrow + row] += rs;
        float* gf = own + 10 * TT + i * BC;                // dQ~ = G_{a-1}, fp32 rows
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 x4 = {g[blk][4 * g4], g[blk][4 * g4 + 1], g[blk][4 * g4 + 2], g[blk][4 * g4 + 3]};
                *reinterpret_cast<f32x4*>(gf + 32 * blk + 8 * g4 + 4 * hh) = x4;
            }
    }
}

// ---------------------------------------------------------------------------
// dQ~ through Q~ = Q - lower(X) U, X = Q W^T (four waves, LDS tiles):
// dQ = dQ_own + dQ~ + dXl W, dXl = dXl_own - lower(dQ~ U^T),
// dU = -lower(X)^T dQ~, dW_own = dXl^T Q.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 2) void path_bwd_own_end_kernel(const BwdKArgs a) {
    __shared__ __attribute__((aligned(16))) bf16 tA[BT], tB[BT], tC[BT], tD[BT], tF[BT], tXT[BT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int L = a.L, N = a.N;
    int head, ca;
    wg_map(blockIdx.x, a.BH, N, false, head, ca);
    const int p0 = ca * BC, nva = min(BC, L - p0);
    const size_t hrow = (size_t)head * L, chunk0 = (size_t)head * N;
    const int n = qcol(wave, lane);
    const bf16* q = static_cast<const bf16*>(a.q) + (hrow + p0) * BC;
    const bf16* w = static_cast<const bf16*>(a.w) + (hrow + p0) * BC;
    const bf16* un = static_cast<const bf16*>(a.ut) + (chunk0 + ca) * TT;
    float* own = a.own + (chunk0 + ca) * NOWN * TT;

    const Frag fq = fetch(q, nva, tid), fw = fetch(w, nva, tid), fu = fetch(un, BC, tid);
    put(tA, fq, tid);                                        // Q [i][d]
    put(tB, fw, tid);                                        // W [m][d]
    __syncthreads();
    {
        f32x16 x = mm_nt(tA, tB, z16(), wave, lane);         // X[i][m]
#pragma unroll
        for (int v = 0; v < 16; ++v)
            if (n > qrow(wave, lane, v)) x[v] = 0.f;
        st_q<true>(tXT, x, wave, lane);                      // lower(X)^T [m][i]
    }
    const f32x16 g = ca >= 1 ? ld_qg(own + 10 * TT, wave, lane) : z16();   // dQ~ [i][e]
    __syncthreads();
    st_q<false>(tA, g, wave, lane);                          // dQ~ [i][e]
    st_q<true>(tB, g, wave, lane);                           // dQ~^T [e][i]
    put(tC, fu, tid);                                        // U [m][e]
    put_t(tD, fw, tid);                                      // W^T [d][m]
    put_t(tF, fq, tid);                                      // Q^T [d][i]
    __syncthreads();
    const f32x16 du = mm_nt(tA, tC, z16(), wave, lane);      // (dQ~ U^T)[i][m]
    f32x16 dq = ld_qg(own + 7 * TT, wave, lane);
    f32x16 dxl = ld_qg(own + 8 * TT, wave, lane);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        dq[v] += g[v];
        dxl[v] -= (n <= qrow(wave, lane, v)) ? du[v] : 0.f;
    }
    st_qg(own + 3 * TT, mm_nt(tXT, tB, z16(), wave, lane), wave, lane, -1.f);   // dU [m][e]
    __syncthreads();
    st_q<false>(tA, dxl, wave, lane);                        // dXl [i][m]
    st_q<true>(tB, dxl, wave, lane);                         // dXl^T [m][i]
    __syncthreads();
    const f32x16 dqw = mm_nt(tA, tD, z16(), wave, lane);     // dXl W
    st_qg(own + 4 * TT, mm_nt(tB, tF, z16(), wave, lane), wave, lane);   // dW_own = dXl^T Q
    float* dqg = a.dq + (hrow + p0) * BC;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int i = qrow(wave, lane, v);
        if (i < nva) dqg[(size_t)i * BC + n] = dq[v] + dqw[v];
    }
}

// ---------------------------------------------------------------------------
// Key chunk b, summed over the query chunks a > b (four waves; wave w holds
// the keys 32 kh .. 32 kh + 31, kh = w & 1, as the columns of its
// accumulators and takes the queries 32 qh .. 32 qh + 31, qh = w >> 1, of
// every query chunk):
//   S = Q_{a,b} K~_b^T, dP = dO_a V_b^T, P, dS (rows = the wave's queries);
//   dV^T += dO_a^T P, dK~^T += Q_{a,b}^T dS, dM += Q_{a,b}^T G_{a,b-1}
// (dM: columns y = the wave's key half).  The k axis of the last three is the
// wave's half of the query axis, in slot order; the two query halves' partial
// sums are added through LDS at the end.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 2) void path_bwd_key_kernel(const BwdKArgs a) {
    // five tiles in one array (the end's reduction reuses it as 16 KB of fp32)
    __shared__ __attribute__((aligned(16))) bf16 tiles[5 * BT];
    __shared__ __attribute__((aligned(16))) float sRq[BC + 4], sD[BC];   // sRq[64]: the pair's gate bias
    bf16* const tQ = tiles;
    bf16* const tQT = tiles + BT;
    bf16* const tO = tiles + 2 * BT;
    bf16* const tOT = tiles + 3 * BT;
    bf16* const tGT = tiles + 4 * BT;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int kh = wave & 1, qh = wave >> 1;       // key half, query half of the wave
    const int L = a.L, N = a.N, Lp = N * BC;
    int head, cb;
    wg_map(blockIdx.x, a.BH, N, false, head, cb);
    const int p0 = cb * BC, nvb = min(BC, L - p0);
    const int j = 32 * kh + l32;                    // the lane's key within the chunk
    const size_t hrow = (size_t)head * L, wrow = (size_t)head * Lp, chunk0 = (size_t)head * N;
    const bool gate = a.loc != nullptr;
    const float c2 = a.scale * kLog2e;
    const size_t pairs = (size_t)N * (N - 1) / 2;
    const bf16* qs = static_cast<const bf16*>(a.qs) + (size_t)head * pairs * TT;
    const bf16* gs = static_cast<const bf16*>(a.gs) + (size_t)head * pairs * TT;
    const bf16* dOg = static_cast<const bf16*>(a.dout) + hrow * BC;
    float* own = a.own + (chunk0 + cb) * NOWN * TT;

    // the key's B operands: K~ (d in slot order, as the stored queries) and V
    bf16x8 kb[4], vb[4];
    {
        const bf16* kr = static_cast<const bf16*>(a.kp) + (chunk0 + cb) * TT + j * BC + 8 * hh;
        const bf16* vr = static_cast<const bf16*>(a.v) + (hrow + p0 + j) * BC + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            kb[ks] = l8(kr + 16 * ks);
            vb[ks] = bf16x8{};
            if (j < nvb) vb[ks] = l8(vr + 16 * ks);
        }
    }
    const float locK = gate ? a.loc[wrow + p0 + j] : 0.f;

    // query chunk ca's tiles and per-query values in flight (raw loads only:
    // they are combined at the stage, where the tiles are waited for anyway)
    Frag fQ = {}, fO = {}, fG = {};
    float lse_n = 0.f, loc_n = 0.f, d_n = 0.f, cs_n = 0.f;
    auto prefetch = [&](int cn) {
        const int pa = cn * BC, nva = min(BC, L - pa);
        fQ = fetch(qs + pair_index(cn, cb) * TT, BC, tid);
        fO = fetch(dOg + (size_t)pa * BC, nva, tid);
        if (cb >= 1) fG = fetch(gs + pair_index(cn, cb) * TT, BC, tid);
        if (tid < BC) {
            lse_n = tid < nva ? a.lse[hrow + pa + tid] : INFINITY;
            loc_n = gate ? a.loc[wrow + pa + tid] : 0.f;
            d_n = a.dsum[wrow + pa + tid];
        }
        if (gate && tid == BC) cs_n = a.csum[chunk0 + cn];
    };
    double fpre = 0.0;              // sum of csum over chunks b+1 .. ca (thread 64)
    if (cb + 1 < N) prefetch(cb + 1);
    // accumulators over the wave's query half: dV^T, dK~^T (rows e, the
    // wave's keys) and dM (rows x, columns y = the wave's key half)
    f32x16 dv[2] = {z16(), z16()}, dk[2] = {z16(), z16()}, dm[2] = {z16(), z16()};
    float cs = 0.f;
    for (int ca = cb + 1; ca < N; ++ca) {
        __syncthreads();
        put(tQ, fQ, tid);                                    // Q_{a,b} [i][slot]
        put_tp(tQT, fQ, tid);                                // Q_{a,b}^T [x][slot of i]
        put(tO, fO, tid);                                    // dO_a [i][d]
        put_to(tOT, fO, tid);                                // dO_a^T [d][slot of i]
        if (cb >= 1) put_tp(tGT, fG, tid);                   // G^T [y][slot of i]
        if (tid < BC) {
            sRq[tid] = loc_n - lse_n * kLog2e;               // -inf past L
            sD[tid] = d_n;
        }
        if (tid == BC) {
            fpre += static_cast<double>(cs_n);
            sRq[BC] = static_cast<float>(fpre);
        }
        __syncthreads();
        if (ca + 1 < N) prefetch(ca + 1);
        // S, dP for queries 32 qh .. +31 (rows) and the wave's keys (columns)
        f32x16 s = z16(), dp = z16();
        {
            const bf16* qa = tQ + (32 * qh + l32) * BP + 8 * hh;
            const bf16* oa = tO + (32 * qh + l32) * BP + 8 * hh;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                s = mfmab(l8(qa + 16 * ks), kb[ks], s);
                dp = mfmab(l8(oa + 16 * ks), vb[ks], dp);
            }
        }
        const float colterm = sRq[BC] - locK;                // bias - the key's gate term
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 rq = *reinterpret_cast<const f32x4*>(sRq + 32 * qh + 8 * g4 + 4 * hh);
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(sD + 32 * qh + 8 * g4 + 4 * hh);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int v = 4 * g4 + r;
                const float p = __builtin_amdgcn_exp2f(c2 * s[v] + rq[r] + colterm);
                const float d = p * (dp[v] - d4[r]);
                cs += d;
                s[v] = p;
                dp[v] = d;
            }
        }
        // the k axis of the next products is the wave's 32 query slots:
        // k-steps 2 qh and 2 qh + 1 of the 64-slot axis
        const bf16x8 pb0 = cvt8<0>(s), pb1 = cvt8<1>(s);
        const bf16x8 db0 = cvt8<0>(dp), db1 = cvt8<1>(dp);
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            dv[blk] = mfmab(aop(tOT, blk, 2 * qh, lane), pb0, dv[blk]);
            dv[blk] = mfmab(aop(tOT, blk, 2 * qh + 1, lane), pb1, dv[blk]);
            const bf16x8 aq0 = aop(tQT, blk, 2 * qh, lane), aq1 = aop(tQT, blk, 2 * qh + 1, lane);
            dk[blk] = mfmab(aq0, db0, dk[blk]);
            dk[blk] = mfmab(aq1, db1, dk[blk]);
            if (cb >= 1) {
                const bf16* gr = tGT + j * BP + 32 * qh + 8 * hh;
                dm[blk] = mfmab(aq0, l8(gr), dm[blk]);
                dm[blk] = mfmab(aq1, l8(gr + 16), dm[blk]);
            }
        }
    }
    // Sum the two query halves through LDS (waves 2, 3 hand their partials to
    // waves 0, 1), then: dV = the later queries' part + the own chunk's; dK~
    // (scaled) and dM for the UT kernel; the column sums of dS.
    float* red = reinterpret_cast<float*>(tiles);           // 2 x 2 x 16 x 64 floats per pass
    auto reduce = [&](f32x16* acc) {
        __syncthreads();
        if (qh == 1)
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int v = 0; v < 16; ++v) red[((kh * 2 + blk) * 16 + v) * 64 + lane] = acc[blk][v];
        __syncthreads();
        if (qh == 0)
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[blk][v] += red[((kh * 2 + blk) * 16 + v) * 64 + lane];
    };
    reduce(dv);
    reduce(dk);
    reduce(dm);
    __syncthreads();
    if (qh == 1) red[kh * 64 + lane] = cs;
    __syncthreads();
    if (qh == 0) {
        cs += red[kh * 64 + lane];
        const float* dvo = own + 1 * TT + j * BC;
        float* dvg = a.dv + (hrow + p0 + j) * BC;
        float* dkt = own + 5 * TT + j * BC;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int e = 32 * blk + 8 * g4 + 4 * hh;
                const f32x4 o4 = *reinterpret_cast<const f32x4*>(dvo + e);
                const f32x4 v4 = {dv[blk][4 * g4] + o4[0], dv[blk][4 * g4 + 1] + o4[1],
                                  dv[blk][4 * g4 + 2] + o4[2], dv[blk][4 * g4 + 3] + o4[3]};
                if (j < nvb) *reinterpret_cast<f32x4*>(dvg + e) = v4;
                const f32x4 k4 = {a.scale * dk[blk][4 * g4], a.scale * dk[blk][4 * g4 + 1],
                                  a.scale * dk[blk][4 * g4 + 2], a.scale * dk[blk][4 * g4 + 3]};
                *reinterpret_cast<f32x4*>(dkt + e) = k4;
            }
        float* dmg = own + 6 * TT;                           // dM[x][y] = -(Q^T G)[x][y]
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                dmg[(32 * blk + 8 * (v >> 2) + 4 * hh + (v & 3)) * BC + j] = -dm[blk][v];
        cs += __shfl_xor(cs, 32, 64);
        if (hh == 0) a.csl[wrow + p0 + j] = cs;
    }
}

// ---------------------------------------------------------------------------
// UT-transform backward of one chunk.  Inputs: dK~, dM (key kernel) and
// dU, dY, the own-chunk dK, dW (query kernel).  Recomputed: G = W W^T,
// X = (I + A)^{-1} with A = strictLower(D G), T^{-1} = X D,
// R = strictLower(W K^T), Y = T^{-1} R, U = T^{-1} W.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 2) void path_bwd_ut_kernel(const BwdKArgs a) {
    // Eight tiles in one array.  Until T^{-1} is formed, the fp32 G and
    // X = (I + A)^{-1} of the substitution live over tE, tF and tH, tI; each
    // wave then keeps its 32 x 32 quarters of G and X in registers, which is
    // all that later steps read of them.  74 KB: two workgroups per CU.
    __shared__ __attribute__((aligned(16))) bf16 tiles[8 * BT];
    __shared__ float sB[BC], sDb[BC];
    bf16* const tA = tiles;
    bf16* const tB = tiles + BT;
    bf16* const tCt = tiles + 2 * BT;
    bf16* const tD = tiles + 3 * BT;
    bf16* const tE = tiles + 4 * BT;
    bf16* const tF = tiles + 5 * BT;
    bf16* const tH = tiles + 6 * BT;
    bf16* const tI = tiles + 7 * BT;
    float* const sG = reinterpret_cast<float*>(tE);        // [64][FP] over tE, tF
    float* const sX = reinterpret_cast<float*>(tH);        // [64][FP] over tH, tI
    static_assert(BC * FP * 4 <= 2 * BT * 2, "fp32 tile over two bf16 tiles");

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
    const f32x16 gq = mm_nt(tA, tA, z16(), wave, lane);             // G = W W^T (kept)
#pragma unroll
    for (int v = 0; v < 16; ++v) sG[qrow(wave, lane, v) * FP + n] = gq[v];
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
            float acc[4] = {0.f, 0.f, 0.f, 0.f};          // four independent chains
#pragma unroll
            for (int p = 0; p < m; ++p) acc[p & 3] = fmaf(grow[p], t[p], acc[p & 3]);
            t[m] = (m == lane ? 1.f : 0.f) - sB[m] * ((acc[0] + acc[1]) + (acc[2] + acc[3]));
        }
#pragma unroll
        for (int m = 0; m < BC; ++m) sX[m * FP + lane] = t[m];
    }
    __syncthreads();
    f32x16 xq;                                                       // the wave's quarter of X
#pragma unroll
    for (int v = 0; v < 16; ++v) xq[v] = sX[qrow(wave, lane, v) * FP + n];
    for (int u = tid; u < BC * BC; u += 256) {                      // T^{-1} = X D (over sG)
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
    // dR = T^{-T} dY (strictly lower), dW += T^{-T} dU.  These products and
    // those of dA below take their factors as hi + lo bf16 pairs (about 16
    // bits): with transitions close to one another and beta near 2 (I + A
    // ill-conditioned) single bf16 roundings of T^{-1}, dY, dU, X, dX and
    // Z left several per cent of error in dW, dK and dbeta.
    __syncthreads();
    st_q2<true>(tH, tA, dY, wave, lane);                             // dY^T [j][m] (W rows no longer read)
    st_q2<true>(tI, tCt, dU, wave, lane);                            // dU^T [e][m]
    st_q2<true>(tF, tE, xq, wave, lane, sB[n]);                      // T^{-T} [n][m], hi over the same values
    __syncthreads();
    f32x16 dR = mm_nt3(tF, tE, tH, tA, z16(), wave, lane);          // [n][j]
#pragma unroll
    for (int v = 0; v < 16; ++v)
        if (qrow(wave, lane, v) <= n) dR[v] = 0.f;
    {
        const f32x16 t1 = mm_nt3(tF, tE, tI, tCt, z16(), wave, lane);   // T^{-T} dU [n][e]
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
            dX[v] = dT[v] * sB[n];
            cs += xq[v] * dT[v];
        }
        cs += __shfl_xor(cs, 32, 64);
        if (lane < 32) atomicAdd(&sDb[n], cs);
    }
    // X = (I + A)^{-1}: dA = -X^T dX X^T via Z = dX X^T, dA = -X^T Z
    // (hi + lo factors; tA, tD, tE are free again)
    __syncthreads();
    st_q2<false>(tH, tA, dX, wave, lane);                            // dX [m][c]
    st_q2<false>(tI, tD, xq, wave, lane);                            // X [p][c]
    st_q2<true>(tCt, tE, xq, wave, lane);                            // X^T [c][m]
    __syncthreads();
    const f32x16 zq = mm_nt3(tH, tA, tI, tD, z16(), wave, lane);    // Z = dX X^T [m][p]
    __syncthreads();
    st_q2<true>(tH, tA, zq, wave, lane);                             // Z^T [p][m]
    __syncthreads();
    f32x16 dA = mm_nt3(tCt, tE, tH, tA, z16(), wave, lane);         // X^T Z [q][p]
    // A = strictLower(D G): dbeta_q += sum_{p<q} dA[q][p] G[q][p], dG = beta_q dA
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int qr = qrow(wave, lane, v);
        const float da = (n < qr) ? -dA[v] : 0.f;
        dA[v] = sB[qr] * da;
        const float r = wave_sum32(da * gq[v]);
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
    const dim3 grid(a.BH * a.N);
    hipLaunchKernelGGL(path_bwd_layout_kernel, grid, dim3(256), 0, s, a);
    hipLaunchKernelGGL(path_bwd_own_kernel, grid, dim3(256), 0, s, a);
    if (a.N >= 2) hipLaunchKernelGGL(path_bwd_chain_kernel, dim3(a.BH * (a.N / 2)), dim3(256), 0, s, a);
    hipLaunchKernelGGL(path_bwd_own_end_kernel, grid, dim3(256), 0, s, a);
    hipLaunchKernelGGL(path_bwd_key_kernel, grid, dim3(256), 0, s, a);
    hipLaunchKernelGGL(path_bwd_ut_kernel, grid, dim3(256), 0, s, a);
    if (a.log_f) hipLaunchKernelGGL(path_bwd_gate_kernel, dim3(a.BH), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace path
