// path_fwd (bf16 mode): blockwise PaTH attention forward on gfx950 MFMA,
// the right-to-left scan over key chunks.
//
// Algorithm (Dutch summary section 3: boundary-adjusted queries/keys per
// block, a right-to-left scan over key/value blocks, FlashAttention-style
// on-chip tiling; Chinese notes, training strategy: UT transform and the
// full-matrix form).  Chunks hold C = 64 tokens.  A query chunk a walks the
// key chunks b = a, a-1, ..., 0:
//   b = a:  S = Q K~^T + strictUpper(Q W^T) Y   (causal mask j <= i)
//           Q <- Q - lower(Q W^T) U             (query carried to chunk start)
//   b < a:  S = Q K~^T;  Q carried through chunk b
// and accumulates softmax(S) V online.  The step b = a is taken by the
// prepare stage (path_ut_bf16.hip), which leaves the query carried to its
// chunk start, the pending probabilities of its own keys and their maximum
// and sum.  This scan carries the query through every left chunk with the
// chunk's d x d product, Q <- Q - Q M (M = W^T U): 2 d^2 flops per query and
// chunk, against 4 C d for the rank-C form Q - (Q W^T) U (half at d = 64,
// the same at d = 128, with one operand tile per chunk instead of two).
// Every product is a bf16 MFMA with fp32 accumulation; the carried query Q
// stays in fp32 accumulators and is rounded to bf16 only as an MFMA operand.
//
// Kernels: path_fwd_bf16_d64pp_kernel (d = 64) and
// path_fwd_bf16_d128pp_kernel (d = 128).  A workgroup of 8 waves (two per
// SIMD, in alternating matrix and vector phases) holds four query chunks;
// workgroups are persistent, one per CU.
//
// Orientation.  All products are formed transposed (S^T = K~ Q^T,
// O^T += V^T P^T, Q^T += (-M^T) Q^T), so every accumulator
// that feeds a later product (S^T -> P^T, Q^T) is already in B-operand
// position: accumulator registers 8s..8s+7 are the B operand of k-step s
// under the k-slot permutation perm16 (path_internal.h).  The transposed
// tiles the prepare stage writes have their key axis in that slot order and
// their d rows permuted, so the carried query and the output come out with d
// in natural order, and every LDS operand read is one 16-byte ds_read (or,
// for the d = 64 V tile, LDS transpose loads).
//
// Staging.  Key chunks are copied HBM/L2 -> LDS with global_load_lds (no
// VGPRs) into two alternating stage sets while the waves compute on the
// other.  LDS tiles are unpadded, their 16-byte units XOR-swizzled per row.
// Dealing: pairs of query blocks of equal total work, and when B*H is a
// multiple of 8 all blocks of one head go to one XCD, so a head's chunks are
// reused out of that XCD's L2.
#include <type_traits>

#include "path_internal.h"

namespace path {

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// accumulator registers 8*half .. 8*half+7 as a bf16 B operand
__device__ __forceinline__ bf16x8 pack8(const f32x16& acc, int half) {
    bf16x8 r;
#pragma unroll
    for (int t = 0; t < 8; ++t) r[t] = static_cast<bf16>(acc[8 * half + t]);
    return r;
}

__device__ __forceinline__ bf16x8 lds8(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

typedef __attribute__((address_space(3))) void lds_void;

// The PV A operands of the d = 64 V tile (kept as it is, [64 tokens][64 d])
// come from LDS transpose loads: swz_v, vtr_offsets and pv_operand in
// path_internal.h.
typedef __attribute__((address_space(1))) const void gbl_void;

// Swizzled tile: 16-byte unit u of row r sits at unit u ^ g(r).  g keeps the
// 32-row MFMA operand reads (16-byte per lane, consecutive lanes on
// consecutive rows) on distinct banks whether the LDS serves 8 or 16 lanes
// per cycle: rows of 128 bytes use g(r) = (r ^ ((r >> 3) & 3)) & 7, rows of
// 256 bytes use g(r) = r & 15.  Both repeat every 32 rows, so a lane reading
// rows 32t + lane%32 uses one offset for every t.
template <int COLS>
__device__ __forceinline__ int swz_g(int r) {
    return COLS == 64 ? ((r ^ ((r >> 3) & 3)) & 7) : (r & 15);
}

// Synchronous guarded copy (rows >= nvalid are zero) into a swizzled tile by
// NT threads; VTILE: the V tile's swizzle.
template <int ROWS, int COLS, int NT = 256, bool VTILE = false>
__device__ __forceinline__ void copy_guarded(bf16* lds, const bf16* g, int nvalid, int tid) {
    constexpr int UPR = COLS / 8;
#pragma unroll
    for (int i = tid; i < ROWS * UPR; i += NT) {
        const int r = i / UPR, u = i % UPR;
        uint4 val = {0u, 0u, 0u, 0u};
        if (r < nvalid) val = *reinterpret_cast<const uint4*>(g + (size_t)r * COLS + u * 8);
        const int x = VTILE ? swz_v(r) : swz_g<COLS>(r);
        *reinterpret_cast<uint4*>(lds + r * COLS + ((u ^ x) << 3)) = val;
    }
}

// Copies of a contiguous [64][64] bf16 tile (8 KB) into a swizzled LDS tile
// by 8 waves: wave w fills the 1 KB block w (rows 8w .. 8w+7, lane i -> LDS
// bytes 16i .. 16i+15), its lane reading the global unit that belongs there.
// Both swizzles depend on the row's low 3 bits only, so the offset is the
// same for every tile of the kind.
__device__ __forceinline__ unsigned tile64_lane_offset(int wave, int lane) {
    const int r = 8 * wave + (lane >> 3);
    const int u = (lane & 7) ^ swz_g<64>(r);
    return static_cast<unsigned>((r * 64 + u * 8) * 2);
}
__device__ __forceinline__ unsigned vtile_lane_offset(int wave, int lane) {
    const int r = 8 * wave + (lane >> 3);
    const int u = (lane & 7) ^ swz_v(r);
    return static_cast<unsigned>((r * 64 + u * 8) * 2);
}

__device__ __forceinline__ void wait_vmem() {
    __builtin_amdgcn_s_waitcnt(0x0f70);       // vmcnt(0)
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum of a value with the lane 32 positions away (the two lane halves
// hold the two key halves of the same query column)
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, bool GATE>
struct WaveState {
    static constexpr int DT = D / 32, KSD = D / 16;
    f32x16 qacc[DT];   // carried query Q^T (fp32); register 8s+t = d 32dt+16s+8hh+t
    bf16x8 qB[KSD];    // its bf16 B operand (d = 64; at d = 128 it is packed where used)
    f32x16 oacc[DT];   // O^T (unnormalised), same d mapping
    float m_run, l_run, loc_i;
    double dab;        // gate: sum of chunk sums between the query chunk and the key chunk
    int offD[KSD];     // swizzled offsets of unit 2ks+hh in a D-wide row  (row = 32x + lane%32)
    int offC_[D == 64 ? 1 : 4];   // same in a 64-wide row, k-steps 0..3 (d = 64: equal to offD)
    unsigned voff[D == 64 ? 8 : 1]; // d = 64: transpose-load offsets of the PV operands
    unsigned lb, lbv;  // d = 128: byte offset of the lane's k-step 0 unit in a 256-byte
                       // (lb) and a 128-byte (lbv) row tile, rows 32x + lane%32
    __device__ __forceinline__ int offC(int ks) const { return D == 64 ? offD[ks] : offC_[ks]; }
};

template <int D>
struct Stage {
    bf16* k;           // K~  [C][D]
    bf16* v;           // V   [C][D] (d = 64: read with transpose loads)
    bf16* mt;          // -M^T [D][D]
    float* loc;        // -local log2 gate prefix [C], then the chunk's gate sum
    bf16* gb;          // with gate: bias k-step A rows [C][16]
};

// Three-term bf16 split, x = h + m + l to about 24 bits.
__device__ __forceinline__ void split3(float x, bf16& h, bf16& m, bf16& l) {
    h = static_cast<bf16>(x);
    const float r = x - static_cast<float>(h);
    m = static_cast<bf16>(r);
    l = static_cast<bf16>(r - static_cast<float>(m));
}

// x with every 32-bit lane word ANDed with msk (0 or ~0)
__device__ __forceinline__ bf16x8 mask8(bf16x8 x, unsigned msk) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    u32x4 w = __builtin_bit_cast(u32x4, x);
    w &= msk;
    return __builtin_bit_cast(bf16x8, w);
}

// Row sums above this trigger a rescale in the d = 64 key-chunk step (the
// probabilities are then bounded by it before the final normalisation).
constexpr float kRescaleTrigger = 4096.f;

// Probabilities of one 32-key tile (accumulator registers 0..15 = two PV
// k-steps), summed as the rounded values the PV product uses.
__device__ __forceinline__ float tile_probs(const f32x16& s, bf16x8& p0, bf16x8& p1, float shift) {
    const bf16 one = static_cast<bf16>(1.f);
    float sum = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) p0[t] = static_cast<bf16>(fast_exp2(s[t] - shift));
#pragma unroll
    for (int t = 0; t < 8; ++t) p1[t] = static_cast<bf16>(fast_exp2(s[8 + t] - shift));
#pragma unroll
    for (int t = 0; t < 8; t += 2) sum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p0[t], p0[t + 1]}, bf16x2{one, one}, sum, false);
#pragma unroll
    for (int t = 0; t < 8; t += 2) sum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p1[t], p1[t + 1]}, bf16x2{one, one}, sum, false);
    return sum;
}

__device__ __forceinline__ float tile_max(const f32x16& s) {
    float mx = s[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = fmaxf(mx, s[v]);
    return mx;
}

// Raise the running maximum by shift >= 0: rescale O and l.
template <int D, bool GATE>
__device__ __forceinline__ void raise_max(WaveState<D, GATE>& st, float shift) {
    const float alpha = fast_exp2(-shift);
    st.m_run += shift;
    st.l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) st.oacc[dt][v] *= alpha;
}

// A wave's query block, query chunk and row within it.
template <int D, bool GATE>
struct ScanSetup {
    int head, qb, qc, iloc, qi;
    bool active, qvalid;
};

// Normalised output row and log-sum-exp (natural log).
template <int D, bool GATE>
__device__ __forceinline__ void scan_store(const FwdArgs& a, const WaveState<D, GATE>& st,
                                           const ScanSetup<D, GATE>& u, int hh) {
    constexpr int KSD = D / 16;
    if (!u.active) return;
    const float l_tot = pair_sum(st.l_run);
    if (!u.qvalid) return;
    const float inv = 1.f / l_tot;
    bf16* orow = static_cast<bf16*>(a.out) + ((size_t)u.head * a.L + u.qi) * D;
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
        bf16x8 o8;
#pragma unroll
        for (int t = 0; t < 8; ++t) o8[t] = static_cast<bf16>(st.oacc[ks >> 1][8 * (ks & 1) + t] * inv);
        *reinterpret_cast<bf16x8*>(orow + 16 * ks + 8 * hh) = o8;
    }
    if (a.lse && hh == 0) a.lse[(size_t)u.head * a.L + u.qi] = (st.m_run + log2f(l_tot)) * kLn2;
}

// ---------------------------------------------------------------------------
// d = 64, two waves per SIMD in alternating phases.
//
// A workgroup of 8 waves holds query chunks 4qb .. 4qb+3 of one head; wave w
// runs on SIMD w % 4 (the hardware deals a workgroup's waves to the SIMDs in
// turn).  Query chunk 4qb + j is split between waves j and 7 - j, on two
// different SIMDs.  Each wave starts from the prepare stage's state after its
// own chunk (the query carried to the chunk start, the pending probabilities
// of the own keys, their maximum and sum).  Every key chunk left of its own is
// split per wave into a matrix phase (PV of the previous chunk, logits and
// carry of this one: 26 MFMAs) and a vector phase (the probabilities: 32
// exps).  Waves 4..7 run one phase ahead of waves 0..3 and a workgroup
// barrier separates the phases, so on every SIMD one wave's MFMAs run while
// the other wave's vector instructions issue.
//
// Staging: a key chunk's K~, -M^T, V, gate rows and sums sit in stage set
// k % 2 and are copied two phases before their first use.  A workgroup's
// next query block is known in advance: its starting state (each wave's 32
// query rows) and its first key step's tiles are copied into LDS during the
// current block's last phases, so a block starts without a trip to memory.
// ---------------------------------------------------------------------------

// Matrix phase of one wave: O^T += V^T P^T for the pending probabilities pB
// (V tile sv), then with QK the carried query's bf16 operand (packed from its
// accumulator under the PV MFMAs), the logits of the staged chunk sg (left in
// s as z - m_run), and the -M^T operands of the chunk's carry read into opm (the
// carry's MFMAs are issued in the vector phase, where they fill the matrix
// pipe while the other wave of the SIMD issues the next logits).
//
// The carried query is held pre-scaled by c2 = scale*log2(e) (the transport
// is linear, so this is the same as scaling the logits).  One extra k-step of
// the logit product adds the key's gate term -loc_j and the query's offset
// a_i - m_run, each as three bf16 terms:
//     A row j    = (g_h, g_m, g_l, 1, 1, 1, 0, 0 | 0 ... 0),   g = -loc_j
//     B column i = (1, 1, 1, o_h, o_m, o_l, 0, 0 | 0 ... 0),   o = a_i - m_run
// so the accumulator holds z_ij - m_run and the probabilities are exp2 of it.
// The A rows are written per key by path_ut (gate) or constant (no gate).
// The query is carried through the whole chunk with the chunk's d x d
// product, Q^T += (-M^T) Q^T (M = W^T U).
//
// Issue order: the PV operands are read first and the logit operands (K~
// rows, bias rows) after them, so that the PV MFMAs cover the latency of the
// latter; the -M^T operands are read in the shadow of the logit MFMAs.
template <bool GATE, bool QK>
__device__ __forceinline__ void pp_mphase(WaveState<64, GATE>& st, f32x16 s[2], const bf16x8 pB[4],
                                          bf16x8 opm[8], const Stage<64>& sg, const bf16* sv, int l32, int hh) {
    constexpr int D = 64, KS = 4;
    const bf16 one = static_cast<bf16>(1.f), nil = static_cast<bf16>(0.f);
    const unsigned lower = hh ? 0u : ~0u;
    bf16x8 opv[2 * KS];
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) opv[KS * dt + ks] = pv_operand(sv, st.voff, dt, ks);
    if (!QK) {
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) st.oacc[dt] = mfma32(opv[KS * dt + ks], pB[ks], st.oacc[dt]);
        return;
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) st.qB[ks] = pack8(st.qacc[ks >> 1], ks & 1);
    bf16x8 opg[2], opk[2 * KS];
    const float csum = GATE ? sg.loc[64] : 0.f;   // the chunk's gate sum, for dab
    if (GATE) {
        opg[0] = lds8(sg.gb + l32 * 16 + 8 * hh);
        opg[1] = lds8(sg.gb + (32 + l32) * 16 + 8 * hh);
    } else {
        opg[0] = opg[1] = mask8(bf16x8{nil, nil, nil, one, one, one, nil, nil}, lower);
    }
#pragma unroll
    for (int kt2 = 0; kt2 < 2; ++kt2)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) opk[KS * kt2 + ks] = lds8(sg.k + (32 * kt2 + l32) * D + st.offD[ks]);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) st.oacc[dt] = mfma32(opv[KS * dt + ks], pB[ks], st.oacc[dt]);
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);               // PV operand reads
    __builtin_amdgcn_sched_group_barrier(0x100, GATE ? 11 : 8, 0);    // logit operand reads, csum
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);                // PV MFMAs
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 bq;
    {
        const float a_i = GATE ? st.loc_i + static_cast<float>(st.dab) : 0.f;
        bf16 h, m, l;
        split3(a_i - st.m_run, h, m, l);
        bq = mask8(bf16x8{one, one, one, h, m, l, nil, nil}, lower);
    }
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) opm[KS * dt + ks] = lds8(sg.mt + (32 * dt + l32) * D + st.offD[ks]);
    // the two 32-key tiles alternate, so no MFMA waits for the one before it
#pragma unroll
    for (int kt2 = 0; kt2 < 2; ++kt2) {
#pragma unroll
        for (int v = 0; v < 16; ++v) s[kt2][v] = 0.f;
        s[kt2] = mfma32(opg[kt2], bq, s[kt2]);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int kt2 = 0; kt2 < 2; ++kt2) s[kt2] = mfma32(opk[KS * kt2 + ks], st.qB[ks], s[kt2]);
    // logit MFMAs with the -M^T reads between them
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    if (GATE) st.dab += static_cast<double>(csum);
}

// Vector phase of one wave: the carry of the query through the chunk,
// Q^T += (-M^T) Q^T (operands opm from the matrix phase), with four of the
// probabilities exp2(z - m_run) of the logits s after each of its eight MFMAs
// (so the exps issue while the other wave of the SIMD keeps the matrix pipe
// busy), then the row sums (raising the running maximum and recomputing the
// probabilities when a row sum passes kRescaleTrigger).  The carried query's
// new operand is packed at the start of the next matrix phase, under its PV
// MFMAs.
template <bool GATE>
__device__ __forceinline__ void pp_vphase(WaveState<64, GATE>& st, const f32x16 s[2], bf16x8 pB[4],
                                          const bf16x8 opm[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int ks = i >> 1, dt = i & 1;
        st.qacc[dt] = mfma32(opm[4 * dt + ks], st.qB[ks], st.qacc[dt]);
#pragma unroll
        for (int e = 4 * i; e < 4 * i + 4; ++e) pB[e >> 3][e & 7] = static_cast<bf16>(fast_exp2(s[e >> 4][e & 15]));
        __builtin_amdgcn_sched_barrier(0);
    }
    const bf16 one = static_cast<bf16>(1.f);
    float psum = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int t = 0; t < 8; t += 2)
            psum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pB[ks][t], pB[ks][t + 1]}, bf16x2{one, one}, psum, false);
    if (__any(!(psum <= kRescaleTrigger))) {
        const float shift = fmaxf(pair_max(fmaxf(tile_max(s[0]), tile_max(s[1]))), 0.f);
        raise_max<64, GATE>(st, shift);
        psum = tile_probs(s[0], pB[0], pB[1], shift) + tile_probs(s[1], pB[2], pB[3], shift);
    }
    st.l_run += psum;
}

// Workgroup barrier without a memory fence: stage copies stay in flight
// across it (each wave waits for its own copies explicitly); the clobber keeps
// the compiler from moving LDS accesses across it.
__device__ __forceinline__ void phase_barrier() { asm volatile("s_barrier" ::: "memory"); }

// global -> LDS copies as global_load_lds does them (lane i: 16 or 4 bytes
// from gbase + voff to lds + 16i or 4i), but issued as inline assembly: the
// compiler then neither tracks them nor adds waits for them, so the caller
// must wait (vmcnt) before the data is read.  gbase and lds are wave-uniform.
// The copy takes its LDS base from M0: the assembly sets M0, leaves one wait
// state before the copy, and restores M0 afterwards (the compiler keeps M0
// for itself).
__device__ __forceinline__ unsigned lds_addr(const void* p) {
    return static_cast<unsigned>(reinterpret_cast<uintptr_t>((const lds_void*)p));
}
__device__ __forceinline__ void dma_lds16(const void* gbase, unsigned voff, const void* lds) {
    unsigned keep;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
                 : "=&s"(keep) : "v"(voff), "s"(gbase), "s"(lds_addr(lds)) : "memory");
}
__device__ __forceinline__ void dma_lds4(const void* gbase, unsigned voff, const void* lds) {
    unsigned keep;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
                 "global_load_lds_dword %1, %2\n\ts_mov_b32 m0, %0"
                 : "=&s"(keep) : "v"(voff), "s"(gbase), "s"(lds_addr(lds)) : "memory");
}

template <bool GATE>
__global__ __launch_bounds__(512, 1) void path_fwd_bf16_d64pp_kernel(const FwdArgs a) {
    constexpr int C = 64, D = 64, NT = 512;
    constexpr int TILE = C * D;
    // Two stage sets, each one LDS object for a key chunk's K~, -M^T, V, bias
    // rows and gate terms (the compiler tells copy targets in flight from
    // tiles being read per object, and it tracks only a few objects).
    struct ChunkTiles {
        bf16 k[TILE];
        bf16 m[TILE];
        bf16 v[TILE];
        bf16 gb[GATE ? C * 16 : 8];
        float loc[C + 4];
    };
    // The starting state of a query block, one part per wave (its 32 query
    // rows): the carried query and the pending probabilities (128-byte rows,
    // swizzled like the K~ tile), (m, l) per row, and with the gate each row's
    // loc and the query chunk's sum.  It is copied during the previous block.
    struct BlockState {
        bf16 q[8][32 * D];
        bf16 p[8][32 * C];
        float ml[8][64];
        float loc[8][64];
    };
    // one LDS object, the stage sets first: the loop's reads of them then
    // take their offsets from the instruction's 16-bit offset field
    struct Shared {
        ChunkTiles km0, km1;
        BlockState bs;
    };
    __shared__ __attribute__((aligned(1024))) Shared sh;

    const int wave_u = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const bool leader = wave_u >= 4;
    const int nqb = (a.N + 3) / 4;

    // Copies that a query block (head, qb) needs before its first key step,
    // each wave issuing its share: its rows' starting state, the tiles of
    // chunk ktop-1 (set (ktop-1) % 2) and, when ktop is odd and chunk ktop
    // full, V(ktop) (set 1).  Issued during the previous block, after the
    // last reads of these buffers (V(ktop) of an even ktop would overwrite
    // V(0), which that block still reads, so the block copies it itself).
    auto prefetch = [=](const FwdArgs& a, const int lane, const int head, const int qb) {
        const int L = a.L, N = a.N, Lp = N * C;
        const int qc = 4 * qb + (leader ? 7 - wave_u : wave_u);
        const bool active = qc < N;
        const size_t row0 = (size_t)head * Lp + (active ? qc * C + (wave_u >> 2) * 32 : 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const unsigned off = tile64_lane_offset(j, lane);
            dma_lds16(static_cast<const bf16*>(a.qt) + row0 * D, off, sh.bs.q[wave_u] + 512 * j);
            dma_lds16(static_cast<const bf16*>(a.pd) + row0 * C, off, sh.bs.p[wave_u] + 512 * j);
        }
        dma_lds4(a.ml + 2 * row0, lane * 4, sh.bs.ml[wave_u]);
        if (GATE) {
            if (lane < 32) dma_lds4(a.loc + row0, lane * 4, sh.bs.loc[wave_u]);
            if (lane == 0) dma_lds4(a.csum + (size_t)head * N + (active ? qc : 0), 0, sh.bs.loc[wave_u] + 32);
        }
        const int ktop = min(4 * qb + 3, N - 1);
        if (ktop >= 1) {
            ChunkTiles& sg = (ktop & 1) ? sh.km0 : sh.km1;
            const int kc = ktop - 1;
            const unsigned loff = tile64_lane_offset(wave_u, lane);
            dma_lds16(static_cast<const bf16*>(a.kt) + ((size_t)head * Lp + kc * C) * D, loff, sg.k + wave_u * 512);
            dma_lds16(static_cast<const bf16*>(a.mt) + ((size_t)head * N + kc) * D * D, loff, sg.m + wave_u * 512);
            if (GATE && wave_u < 2)
                dma_lds16(static_cast<const bf16*>(a.gb) + ((size_t)head * Lp + kc * C) * 16 + wave_u * 512,
                          lane * 16, sg.gb + wave_u * 512);
            if (GATE && wave_u == 2) {
                dma_lds4(a.loc + (size_t)head * Lp + kc * C, lane * 4, sg.loc);
                if (lane == 0) dma_lds4(a.csum + (size_t)head * N + kc, 0, sg.loc + C);
            }
        }
        if ((ktop & 1) && (ktop + 1) * C <= L)
            dma_lds16(static_cast<const bf16*>(a.v) + ((size_t)head * L + (size_t)ktop * C) * D,
                      vtile_lane_offset(wave_u, lane), sh.km1.v + wave_u * 512);
    };

    // One query block (head, qb): query chunks 4qb .. 4qb+3 of one head; the
    // block (nhead, nqb_) follows when has_next.  The arguments and the lane
    // id come in through opaque copies, so that nothing derived from them is
    // kept live from one block to the next.
    auto item = [&](const int head, const int qb, const int nhead, const int nqb_, const bool has_next,
                    const FwdArgs& a, const int lane_in) {
    const int lane = lane_in & 63;
    const int tid = wave_u * 64 + lane;
    const int l32 = lane & 31, hh = lane >> 5;
    const int L = a.L, N = a.N, Lp = N * C;
    const unsigned loff = tile64_lane_offset(wave_u, lane);
    const unsigned vloff = vtile_lane_offset(wave_u, lane);
    // query chunk 4qb + j: waves j (rows 0-31) and 7 - j (rows 32-63), which
    // run on different SIMDs (wave w runs on SIMD w % 4)
    WaveState<D, GATE> st;
    bf16x8 pB[4];
    const int qc = 4 * qb + (leader ? 7 - wave_u : wave_u);
    const int iloc = (wave_u >> 2) * 32 + l32;
    const bool active = qc < N;
    ScanSetup<D, GATE> u;
    u.head = head; u.qb = qb; u.qc = qc; u.iloc = iloc; u.active = active;
    u.qi = qc * C + iloc;
    u.qvalid = active && u.qi < L;

    const bf16* kt = static_cast<const bf16*>(a.kt) + (size_t)head * Lp * D;
    const bf16* vin = static_cast<const bf16*>(a.v) + (size_t)head * L * D;
    const bf16* mtg = static_cast<const bf16*>(a.mt) + (size_t)head * N * D * D;
    const float* locg = GATE ? a.loc + (size_t)head * Lp : nullptr;
    const float* csg = GATE ? a.csum + (size_t)head * N : nullptr;
    const bf16* gbg = GATE ? static_cast<const bf16*>(a.gb) + (size_t)head * Lp * 16 : nullptr;

    const Stage<D> set0{sh.km0.k, sh.km0.v, sh.km0.m, sh.km0.loc, sh.km0.gb};
    const Stage<D> set1{sh.km1.k, sh.km1.v, sh.km1.m, sh.km1.loc, sh.km1.gb};

    // ---- the block's first copies (the previous block, or the workgroup's
    // start, issued them); V(ktop) is copied here when it was not.  ktop =
    // the block's top chunk; chunk k's K~/-M^T/gate terms sit in set k % 2,
    // its V tile in that set's V tile. ----
    const int ktop = min(4 * qb + 3, N - 1);
    wait_vmem();
    if (!((ktop & 1) && (ktop + 1) * C <= L)) {
        bf16* const vtop = (ktop & 1) ? sh.km1.v : sh.km0.v;
        if ((ktop + 1) * C <= L) {
            __builtin_amdgcn_global_load_lds(
                (gbl_void*)(reinterpret_cast<const char*>(vin + (size_t)ktop * TILE) + vloff),
                (lds_void*)(reinterpret_cast<char*>(vtop) + wave_u * 1024), 16, 0, 0);
            wait_vmem();
        } else {
            copy_guarded<C, D, NT, true>(vtop, vin + (size_t)ktop * TILE, L - ktop * C, tid);   // ragged: zero rows
        }
    }
    __syncthreads();
    {
        // the state after the query's own chunk, from the prepare stage: the
        // query carried to its chunk start (scaled by scale*log2(e)), the
        // pending probabilities of its own keys, their maximum and sum
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            st.offD[ks] = ((2 * ks + hh) ^ swz_g<D>(l32)) << 3;
            st.qB[ks] = lds8(sh.bs.q[wave_u] + l32 * D + st.offD[ks]);
            pB[ks] = lds8(sh.bs.p[wave_u] + l32 * C + st.offD[ks]);
#pragma unroll
            for (int t = 0; t < 8; ++t) st.qacc[ks >> 1][8 * (ks & 1) + t] = static_cast<float>(st.qB[ks][t]);
        }
        const f32x2 ml = *reinterpret_cast<const f32x2*>(sh.bs.ml[wave_u] + 2 * l32);
        st.m_run = ml[0];
        st.l_run = hh == 0 ? ml[1] : 0.f;   // the two lane halves' sums are added at the end
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
            for (int v = 0; v < 16; ++v) st.oacc[dt][v] = 0.f;
        st.loc_i = GATE ? sh.bs.loc[wave_u][l32] : 0.f;
        st.dab = GATE ? static_cast<double>(sh.bs.loc[wave_u][32]) : 0.0;
    }
    vtr_offsets(st.voff, lane);

    // ---- key chunks ktop-1 .. 0 in phases.  A wave works on chunk k only
    // when k < qc (its own chunk was done by the prepare stage, whose
    // probabilities are pending against V(qc)); the other waves of the block
    // keep the copies and barriers.  Every wave runs
    //     for k = ktop-1 .. 0:  M(k); barrier; V(k); barrier        then PV(0)
    // where M(k) = PV(k+1), logits and carry of k, and V(k) = the
    // probabilities of k.  The followers (waves 0..3) enter one barrier late,
    // so between two barriers one wave of each SIMD is in a matrix phase and
    // the other in a vector phase.  Copies: at the start of its M(k) a leader
    // issues its blocks of chunk k-1 (K~/-M^T) and V(k); at the start of its
    // V(k) a follower issues its blocks of chunk k-2 and V(k-1), and before
    // the first barrier those of chunk ktop-2 and V(ktop-1) -- the same
    // moment, one phase after the buffers' last reads.  Leaders wait for their
    // copies at the end of V(k), followers at the end of M(k): two phases
    // later, and before the barrier that opens the first phase reading them.
    // The next block's copies are issued once this block's last M(0) is done
    // (by followers at the start of V(0), by leaders after it); then only
    // V(0) is still read. ----
    f32x16 s[2];
    bf16x8 opm[8];
    if (ktop > 0) {
        // copies of the phase loop, issued out of the compiler's sight (it
        // would otherwise pair a copy issued on one role's path with a read
        // on the other's and wait for it); each wave waits for its own.
        auto ktile = [&](bf16* lds, const bf16* g) {
            dma_lds16(g, loff, reinterpret_cast<char*>(lds) + wave_u * 1024);
        };
        auto kissue = [&](const Stage<D>& sg, int kc) {
            ktile(sg.k, kt + (size_t)kc * TILE);
            ktile(sg.mt, mtg + (size_t)kc * TILE);
            if (GATE && wave_u < 2)
                dma_lds16(gbg + (size_t)kc * C * 16 + wave_u * 512, lane * 16, sg.gb + wave_u * 512);
            if (GATE && wave_u == 2) {
                dma_lds4(locg + kc * C, lane * 4, sg.loc);
                if (lane == 0) dma_lds4(csg + kc, 0, sg.loc + C);
            }
        };
        if (!leader) {
            if (ktop >= 2) kissue((ktop & 1) ? set1 : set0, ktop - 2);
            dma_lds16(vin + (size_t)(ktop - 1) * TILE, vloff, ((ktop & 1) ? sh.km0.v : sh.km1.v) + wave_u * 512);
            phase_barrier();
        }
        auto iter = [&](int k, const Stage<D>& ck, const Stage<D>& cn, auto last) {
            // ck: chunk k and V(k); cn: chunk k +- 1 and V(k +- 1).  Chunks
            // below ktop are full, so V is copied without a guard.
            if (leader) {
                if (k >= 1) kissue(cn, k - 1);
                dma_lds16(vin + (size_t)k * TILE, vloff, ck.v + wave_u * 512);
            }
            const bool go = active && k < qc;
            if (go) pp_mphase<GATE, true>(st, s, pB, opm, ck, cn.v, l32, hh);
            if (!leader) wait_vmem();
            phase_barrier();
            if (!leader) {
                if (k >= 2) kissue(ck, k - 2);
                if (k >= 1) dma_lds16(vin + (size_t)(k - 1) * TILE, vloff, cn.v + wave_u * 512);
                if (decltype(last)::value && has_next) prefetch(a, lane, nhead, nqb_);
            }
            if (go) pp_vphase<GATE>(st, s, pB, opm);
            if (leader) wait_vmem();
            phase_barrier();
        };
        // the last step (k = 0) is its own copy: only there do followers
        // issue the next block's copies
        const std::false_type mid;
        const std::true_type last;
        int k = ktop - 1;
        if (k == 0) {
            iter(0, set0, set1, last);
        } else {
            if ((k & 1) == 0) {       // k even: one step to reach the odd/even pairs
                iter(k, set0, set1, mid);
                --k;
            }
            for (; k >= 3; k -= 2) {  // k odd, then k - 1 even
                iter(k, set1, set0, mid);
                iter(k - 1, set0, set1, mid);
            }
            iter(1, set1, set0, mid);
            iter(0, set0, set1, last);
        }
        if (leader && has_next) prefetch(a, lane, nhead, nqb_);
    } else if (has_next) {
        prefetch(a, lane, nhead, nqb_);
    }
    // PV(0) with the pending probabilities (the own chunk's, for qc = 0)
    if (active) pp_mphase<GATE, false>(st, s, pB, opm, set0, set0.v, l32, hh);
    if (ktop > 0 && leader) phase_barrier();
    scan_store<D, GATE>(a, st, u, hh);
    };

    // Persistent workgroups, one per CU.  The query blocks qb and nqb-1-qb of
    // a head together cost the same for every qb (the work of a block grows
    // linearly with qb), so each workgroup takes whole pairs, dealt
    // round-robin.  When BH and the grid are multiples of 8, workgroup b runs
    // on XCD b % 8 (workgroups are dealt to the 8 XCDs in turn) and takes
    // only heads h with h % 8 == b % 8, so a head's chunks are shared in one
    // XCD's L2.
    //
    // When every query block of the launch fits on the CUs at once
    // (a.single), each workgroup takes one block instead: a pair would make
    // the step last a heavy plus a light block while other CUs idle.
    const int G = gridDim.x;
    const int P = (nqb + 1) / 2;                 // pairs per head (an odd nqb leaves one block alone)
    const bool by_xcd = (a.BH % 8) == 0 && (G % 8) == 0;
    const int R = by_xcd ? G / 8 : G;
    const int r = by_xcd ? blockIdx.x / 8 : blockIdx.x;
    const int xcd = by_xcd ? blockIdx.x % 8 : 0;
    const int npairs = (by_xcd ? a.BH / 8 : a.BH) * P;
    const bool single = a.single != 0;
    // the t-th block of this workgroup, t advanced past the lone middle block
    // of an odd nqb: pair r + R (t / 2), heavy half first
    auto deal = [&](int& t, int& head, int& qb) -> bool {
        for (;; ++t) {
            int i;
            if (single) {                        // block r of this workgroup's heads, heaviest first
                if (t > 0) return false;
                i = r / nqb;
                qb = nqb - 1 - r % nqb;
            } else {
                const int j = r + R * (t >> 1);
                if (j >= npairs) return false;
                const int pr = j % P;
                i = j / P;
                qb = (t & 1) ? pr : nqb - 1 - pr;
                if ((t & 1) && qb == nqb - 1 - pr) continue;
            }
            head = by_xcd ? xcd + 8 * i : i;
            return true;
        }
    };
    int t = 0, head = 0, qb = 0;
    bool have = deal(t, head, qb);
    if (have) prefetch(a, static_cast<int>(threadIdx.x & 63), head, qb);
    while (have) {
        int t2 = t + 1, nhead = 0, nqb_ = 0;
        const bool has_next = deal(t2, nhead, nqb_);
        __syncthreads();                         // the previous block's tiles are no longer read
        typedef const __attribute__((address_space(4))) FwdArgs* ArgPtr;
        ArgPtr ap = (ArgPtr)__builtin_amdgcn_kernarg_segment_ptr();
        int ln = static_cast<int>(threadIdx.x & 63);
        asm volatile("" : "+s"(ap), "+v"(ln));
        item(head, qb, nhead, nqb_, has_next, *(const FwdArgs*)ap, ln);
        t = t2; head = nhead; qb = nqb_; have = has_next;
    }
}


// ---------------------------------------------------------------------------
// d = 128, two waves per SIMD in alternating phases.
//
// The workgroup layout, the start from the prepare stage's own-chunk state and
// the persistent dealing are those of the d = 64 kernel; the carry is the
// chunk's d x d product (Q^T += (-M^T) Q^T, 32 MFMAs per wave and chunk, the
// same count as the rank-C form at d = 2C).  A wave's chunk is split as
//     M(k): PV of chunk k+1 (16 MFMAs) and the logits of chunk k (16 + the
//           bias k-step);
//     V(k): the probabilities of chunk k (32 exps), then the carry through
//           chunk k (32 MFMAs, -M^T operands read here),
// so both waves of a SIMD issue MFMAs in every phase.  The staged tiles of
// chunk c sit in set c % 2: K~ (and gate rows) read in M(c), -M^T in V(c),
// V^T of c in M(c-1).  With P(c) the phase of the leaders' M(c), every
// wave issues its share of K~(c-1), the gate rows of c-1 and V^T(c) at the
// start of phase P(c) and of -M^T(c-1) at the start of phase P(c)+1, and
// waits for a phase's copies at the end of the phase after it: each tile's
// slot was last read two phases before its copy must be complete.
// ---------------------------------------------------------------------------

// The byte offset of lane `lane` of wave `wave` in the copy of a tile with
// 256-byte rows (rows of 128 bf16, 16-byte units swizzled by row & 15): one
// wave instruction fills 1 KB of LDS (lane i -> bytes 16i .. 16i+15), i.e.
// rows 4w .. 4w+3 of each 32-row slab; the next slab is 8 KB further in
// both memories and needs the same offset.
__device__ __forceinline__ unsigned tile128_lane_offset(int wave, int lane) {
    const int r = 4 * wave + (lane >> 4);
    const int u = (lane & 15) ^ swz_g<128>(r);
    return static_cast<unsigned>((r * 128 + u * 8) * 2);
}

// vmcnt(n) for the copy counts of the d = 128 phase loop
__device__ __forceinline__ void wait_copies(int n) {
    switch (n) {
        case 0: __builtin_amdgcn_s_waitcnt(0x0f70); break;
        case 2: __builtin_amdgcn_s_waitcnt(0x0f72); break;
        case 4: __builtin_amdgcn_s_waitcnt(0x0f74); break;
        case 5: __builtin_amdgcn_s_waitcnt(0x0f75); break;
        case 6: __builtin_amdgcn_s_waitcnt(0x0f76); break;
        default: __builtin_amdgcn_s_waitcnt(0x0f70); break;
    }
}

template <bool GATE>
struct Tiles128 {
    bf16 k[64 * 128];          // K~ [C][D], natural rows
    bf16 m[128 * 128];         // -M^T [D][D]
    bf16 v[128 * 64];          // V^T [D][C] (128-byte rows, swz_g<64>)
    bf16 gb[GATE ? 64 * 16 : 8];
    float loc[64 + 4];         // [64]: the chunk's gate sum
};

// The phases' MFMAs run as one software-pipelined sequence each: step i
// issues the LDS read of step i + kAhead's A operand, then its own MFMA, and
// a scheduling barrier closes the step, so at most kAhead + 1 operands are in
// registers (the compiler would otherwise hoist every read of the phase and
// run out of registers).
constexpr int kAhead = 3;

// A operand of k-step ks, rows 32 x + lane % 32, in a swizzled tile at byte
// address t: the lane's unit in k-step ks is its k-step-0 unit XOR 2 ks (the
// swizzle is an XOR of the unit index), i.e. byte offset lb ^ 32 ks.
__device__ __forceinline__ bf16x8 tile_op(const void* t, unsigned lb, int ks, int xbytes) {
    return lds8(reinterpret_cast<const bf16*>(static_cast<const char*>(t) + (lb ^ (32u * ks)) + xbytes));
}

// Matrix phase: O^T += V^T P^T for the pending probabilities pB (V^T tile
// sv), then (QK) the logits of chunk ck in s as z - m_run.  Steps 0..15: PV
// (k-step ks = i / 4, row tile dt = i % 4); 16, 17: the start of key tiles 0,
// 1 (with the gate the bias k-step of the d = 64 kernel, else -m_run in
// fp32); 18..33: the logits (k-step (i - 18) / 2, key tile (i - 18) % 2), the
// carried query's operand packed from its fp32 accumulator at its first use.
template <bool GATE, bool QK>
__device__ __forceinline__ void pp128_mphase(WaveState<128, GATE>& st, f32x16 s[2], const bf16x8 pB[4],
                                             const Tiles128<GATE>& ck, const bf16* sv, int l32, int hh) {
    const bf16 one = static_cast<bf16>(1.f), nil = static_cast<bf16>(0.f);
    // per-phase opaque copies: values derived from them (the operand
    // addresses, the constant bias rows) are recomputed in the phase instead
    // of being kept in registers across the loop
    unsigned lower = hh ? 0u : ~0u, lb = st.lb, lbv = st.lbv;
    asm volatile("" : "+v"(lower), "+v"(lb), "+v"(lbv));
    constexpr int NSTEP = QK ? 34 : 16;
    const float csum = (GATE && QK) ? ck.loc[64] : 0.f;
    bf16x8 bq = {};
    if (QK) {
        const float a_i = GATE ? st.loc_i + static_cast<float>(st.dab) : 0.f;
        bf16 h, m, l;
        split3(a_i - st.m_run, h, m, l);
        bq = mask8(bf16x8{one, one, one, h, m, l, nil, nil}, lower);
    }
    const bf16x8 gconst = mask8(bf16x8{nil, nil, nil, one, one, one, nil, nil}, lower);
    auto load = [&](int i) -> bf16x8 {
        if (i < 16) return tile_op(sv, lbv, i >> 2, 4096 * (i & 3));
        if (i < 18) return GATE ? lds8(ck.gb + (32 * (i - 16) + l32) * 16 + 8 * hh) : gconst;
        const int j = i - 18;
        return tile_op(ck.k, lb, j >> 1, 8192 * (j & 1));
    };
    bf16x8 buf[kAhead + 1];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) buf[i] = load(i);
    bf16x8 qb = {};
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
        if (i + kAhead < NSTEP) buf[(i + kAhead) % (kAhead + 1)] = load(i + kAhead);
        const bf16x8 op = buf[i % (kAhead + 1)];
        if (i < 16) {
            st.oacc[i & 3] = mfma32(op, pB[i >> 2], st.oacc[i & 3]);
        } else if (i < 18) {
            f32x16 z;
#pragma unroll
            for (int v = 0; v < 16; ++v) z[v] = GATE ? 0.f : -st.m_run;
            s[i - 16] = GATE ? mfma32(op, bq, z) : z;
        } else {
            const int j = i - 18;
            if ((j & 1) == 0) qb = pack8(st.qacc[j >> 2], (j >> 1) & 1);
            s[j & 1] = mfma32(op, qb, s[j & 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if (GATE && QK) st.dab += static_cast<double>(csum);
}

// Vector phase: the carry through the chunk, Q^T += (-M^T) Q^T (32 steps,
// k-step ks = i / 4, row tile dt = i % 4, the query's eight operands packed
// before the first MFMA changes it), one probability exp2(z - m_run) of the
// logits s per step, then the row sums (raising the running maximum and
// recomputing the probabilities when a row sum passes kRescaleTrigger).
// Spreading the exps over the carry lets them issue while the other wave of
// the SIMD keeps the matrix pipe busy.
template <bool GATE>
__device__ __forceinline__ void pp128_vphase(WaveState<128, GATE>& st, const f32x16 s[2], bf16x8 pB[4],
                                             const bf16* smt) {
    unsigned lb = st.lb;
    asm volatile("" : "+v"(lb));
    auto load = [&](int i) -> bf16x8 { return tile_op(smt, lb, i >> 2, 8192 * (i & 3)); };
    bf16x8 buf[kAhead + 1];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) buf[i] = load(i);
    bf16x8 qb[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qb[ks] = pack8(st.qacc[ks >> 1], ks & 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        if (i + kAhead < 32) buf[(i + kAhead) % (kAhead + 1)] = load(i + kAhead);
        st.qacc[i & 3] = mfma32(buf[i % (kAhead + 1)], qb[i >> 2], st.qacc[i & 3]);
        pB[i >> 3][i & 7] = static_cast<bf16>(fast_exp2(s[i >> 4][i & 15]));
        __builtin_amdgcn_sched_barrier(0);
    }
    const bf16 one = static_cast<bf16>(1.f);
    float psum = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int t = 0; t < 8; t += 2)
            psum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pB[ks][t], pB[ks][t + 1]}, bf16x2{one, one}, psum, false);
    if (__any(!(psum <= kRescaleTrigger))) {
        const float shift = fmaxf(pair_max(fmaxf(tile_max(s[0]), tile_max(s[1]))), 0.f);
        raise_max<128, GATE>(st, shift);
        psum = tile_probs(s[0], pB[0], pB[1], shift) + tile_probs(s[1], pB[2], pB[3], shift);
    }
    st.l_run += psum;
}

template <bool GATE>
__global__ __launch_bounds__(512, 1) void path_fwd_bf16_d128pp_kernel(const FwdArgs a) {
    constexpr int C = 64, D = 128;
    constexpr int KT = C * D;          // K~ and V^T tile elements
    constexpr int MT = D * D;          // -M^T tile elements
    __shared__ __attribute__((aligned(1024))) Tiles128<GATE> km0;
    __shared__ __attribute__((aligned(1024))) Tiles128<GATE> km1;

    const int wave_u = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const bool leader = wave_u >= 4;
    const int nqb = (a.N + 3) / 4;

    auto item = [&](const int head, const int qb, const FwdArgs& a, const int lane_in) {
    const int lane = lane_in & 63;
    const int l32 = lane & 31, hh = lane >> 5;
    const int L = a.L, N = a.N, Lp = N * C;
    const unsigned koff = tile128_lane_offset(wave_u, lane);
    const unsigned voff = tile64_lane_offset(wave_u, lane);
    WaveState<D, GATE> st;
    bf16x8 pB[4];
    const int qc = 4 * qb + (leader ? 7 - wave_u : wave_u);
    const int iloc = (wave_u >> 2) * 32 + l32;
    const bool active = qc < N;
    ScanSetup<D, GATE> u;
    u.head = head; u.qb = qb; u.qc = qc; u.iloc = iloc; u.active = active;
    u.qi = qc * C + iloc;
    u.qvalid = active && u.qi < L;
    {
        // the state after the query's own chunk, from the prepare stage
        const size_t row = (size_t)head * Lp + (active ? u.qi : 0);
        const bf16* qrow = static_cast<const bf16*>(a.qt) + row * D;
        const bf16* prow = static_cast<const bf16*>(a.pd) + row * C;
        st.lb = static_cast<unsigned>(l32 * 256 + 16 * (hh ^ swz_g<D>(l32)));
        st.lbv = static_cast<unsigned>(l32 * 128 + 16 * (hh ^ swz_g<C>(l32)));
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const bf16x8 q8 = lds8(qrow + 16 * ks + 8 * hh);
#pragma unroll
            for (int t = 0; t < 8; ++t) st.qacc[ks >> 1][8 * (ks & 1) + t] = static_cast<float>(q8[t]);
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) pB[ks] = lds8(prow + 16 * ks + 8 * hh);
        const f32x2 ml = *reinterpret_cast<const f32x2*>(a.ml + 2 * row);
        st.m_run = ml[0];
        st.l_run = hh == 0 ? ml[1] : 0.f;   // the two lane halves' sums are added at the end
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int v = 0; v < 16; ++v) st.oacc[dt][v] = 0.f;
        st.loc_i = GATE ? a.loc[row] : 0.f;
        st.dab = GATE ? static_cast<double>(a.csum[(size_t)head * N + (active ? qc : 0)]) : 0.0;
    }

    const char* ktg = static_cast<const char*>(a.kt) + (size_t)head * Lp * D * 2;
    const char* vtg = static_cast<const char*>(a.vt) + (size_t)head * Lp * D * 2;
    const char* mtg = static_cast<const char*>(a.mt) + (size_t)head * N * MT * 2;
    const float* locg = GATE ? a.loc + (size_t)head * Lp : nullptr;
    const float* csg = GATE ? a.csum + (size_t)head * N : nullptr;
    const bf16* gbg = GATE ? static_cast<const bf16*>(a.gb) + (size_t)head * Lp * 16 : nullptr;

    // Copies (every wave its share; the number of copy instructions this wave
    // issued is returned for the wait that follows the next phase).  A(c):
    // K~ and gate rows of chunk c - 1, V^T of chunk c; B(c): -M^T of chunk
    // c - 1.  Chunk c goes to set c % 2.
    auto set_of = [&](int c) -> Tiles128<GATE>& { return (c & 1) ? km1 : km0; };
    auto issue_a = [&](int c) {
        int n = 0;
        if (c >= 1) {
            Tiles128<GATE>& t = set_of(c - 1);
            const char* g = ktg + (size_t)(c - 1) * KT * 2;
#pragma unroll
            for (int j = 0; j < 2; ++j) dma_lds16(g + 8192 * j, koff, reinterpret_cast<char*>(t.k) + 8192 * j + 1024 * wave_u);
            n += 2;
            if (GATE && wave_u < 2) {
                dma_lds16(gbg + (size_t)(c - 1) * C * 16 + wave_u * 512, lane * 16, t.gb + wave_u * 512);
                n += 1;
            }
            if (GATE && wave_u == 2) {
                dma_lds4(locg + (c - 1) * C, lane * 4, t.loc);
                if (lane == 0) dma_lds4(csg + (c - 1), 0, t.loc + C);
                n += 2;
            }
        }
        if (c >= 0) {
            Tiles128<GATE>& t = set_of(c);
            const char* g = vtg + (size_t)c * KT * 2;
#pragma unroll
            for (int j = 0; j < 2; ++j) dma_lds16(g + 8192 * j, voff, reinterpret_cast<char*>(t.v) + 8192 * j + 1024 * wave_u);
            n += 2;
        }
        return n;
    };
    auto issue_b = [&](int c) {
        if (c < 1) return 0;
        Tiles128<GATE>& t = set_of(c - 1);
        const char* g = mtg + (size_t)(c - 1) * MT * 2;
#pragma unroll
        for (int j = 0; j < 4; ++j) dma_lds16(g + 8192 * j, koff, reinterpret_cast<char*>(t.m) + 8192 * j + 1024 * wave_u);
        return 4;
    };

    // ---- key chunks ktop-1 .. 0 in phases, ktop = the block's top chunk.
    // Every wave runs  for k = ktop-1 .. 0:  M(k); barrier; V(k); barrier,
    // then PV(0); the followers (waves 0..3) enter one barrier late.  A
    // leader issues A(k) in M(k) and B(k) in V(k); a follower B(k) in M(k)
    // and A(k-1) in V(k).  The prologue stages A(ktop) and B(ktop). ----
    const int ktop = min(4 * qb + 3, N - 1);
    issue_a(ktop);
    issue_b(ktop);
    wait_vmem();
    __syncthreads();
    f32x16 s[2];
    if (ktop > 0) {
        if (!leader) {
            wait_copies(issue_a(ktop - 1));
            phase_barrier();
        }
        auto iter = [&](int k, const Tiles128<GATE>& ck, const Tiles128<GATE>& cn) {
            // ck: chunk k (K~, -M^T) and V^T(k); cn: V^T(k + 1)
            const bool go = active && k < qc;
            int n = leader ? issue_a(k) : issue_b(k);
            if (go) pp128_mphase<GATE, true>(st, s, pB, ck, cn.v, l32, hh);
            wait_copies(n);
            phase_barrier();
            n = leader ? issue_b(k) : issue_a(k - 1);
            if (go) pp128_vphase<GATE>(st, s, pB, ck.m);
            wait_copies(n);
            phase_barrier();
        };
        int k = ktop - 1;
        if ((k & 1) == 0) {
            iter(k, km0, km1);
            --k;
        }
        for (; k >= 0; k -= 2) {
            iter(k, km1, km0);
            iter(k - 1, km0, km1);
        }
    }
    // PV(0) with the pending probabilities (the own chunk's, for qc = 0)
    if (active) pp128_mphase<GATE, false>(st, s, pB, km0, km0.v, l32, hh);
    if (ktop > 0 && leader) phase_barrier();
    scan_store<D, GATE>(a, st, u, hh);
    };

    // Persistent workgroups: the dealing of the d = 64 kernel.
    const int G = gridDim.x;
    const int P = (nqb + 1) / 2;
    const bool by_xcd = (a.BH % 8) == 0 && (G % 8) == 0;
    const int R = by_xcd ? G / 8 : G;
    const int r = by_xcd ? blockIdx.x / 8 : blockIdx.x;
    const int xcd = by_xcd ? blockIdx.x % 8 : 0;
    const int npairs = (by_xcd ? a.BH / 8 : a.BH) * P;
    const bool single = a.single != 0;
    for (int t = 0;; ++t) {
        int i, qb;
        if (single) {
            if (t > 0) break;
            i = r / nqb;
            qb = nqb - 1 - r % nqb;
        } else {
            const int j = r + R * (t >> 1);
            if (j >= npairs) break;
            const int pr = j % P;
            i = j / P;
            qb = (t & 1) ? pr : nqb - 1 - pr;
            if ((t & 1) && qb == nqb - 1 - pr) continue;
        }
        __syncthreads();
        typedef const __attribute__((address_space(4))) FwdArgs* ArgPtr;
        ArgPtr ap = (ArgPtr)__builtin_amdgcn_kernarg_segment_ptr();
        int ln = static_cast<int>(threadIdx.x & 63);
        asm volatile("" : "+s"(ap), "+v"(ln));
        item(by_xcd ? xcd + 8 * i : i, qb, *(const FwdArgs*)ap, ln);
    }
}

hipError_t launch_path_fwd_bf16(const FwdArgs& args, bool gate, hipStream_t s) {
    FwdArgs a = args;
    if (a.D == 64 || a.D == 128) {
        // persistent: one workgroup per CU (at most one per pair of query
        // blocks), or one per query block when all of them fit at once
        int dev = 0, ncu = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        const long nqb4 = (a.N + 3) / 4;
        const long blocks = (long)a.BH * nqb4;
        const long pairs = (long)a.BH * ((nqb4 + 1) / 2);
        a.single = blocks <= ncu ? 1 : 0;
        long g = a.single ? blocks : (ncu < pairs ? ncu : pairs);
        if (!a.single && g >= 8 && a.BH % 8 == 0) g -= g % 8;
        const dim3 gridp(static_cast<unsigned>(g)), block8(512);
        if (a.D == 64) {
            if (gate) hipLaunchKernelGGL((path_fwd_bf16_d64pp_kernel<true>), gridp, block8, 0, s, a);
            else hipLaunchKernelGGL((path_fwd_bf16_d64pp_kernel<false>), gridp, block8, 0, s, a);
        } else {
            if (gate) hipLaunchKernelGGL((path_fwd_bf16_d128pp_kernel<true>), gridp, block8, 0, s, a);
            else hipLaunchKernelGGL((path_fwd_bf16_d128pp_kernel<false>), gridp, block8, 0, s, a);
        }
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace path
