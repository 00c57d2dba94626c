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
//   b < a:  S = Q K~^T;  Q carried through chunk b (skipped for b = 0)
// and accumulates softmax(S) V online.  Every product is a bf16 MFMA with
// fp32 accumulation; the carried query Q stays in fp32 accumulators and is
// rounded to bf16 only as an MFMA operand.
//
// d = 64 (path_fwd_bf16_d64pp_kernel): the step b = a is taken by the prepare
// stage (path_ut_bf16.hip), which leaves the query carried to its chunk
// start, the pending probabilities of its own keys and their maximum and sum.
// The scan carries the query through every left chunk with the chunk's d x d
// product, Q <- Q - Q M (M = W^T U): 2 d^2 flops per query and chunk against
// 4 C d for the rank-C form.  A workgroup of 8 waves (two per SIMD, in
// alternating matrix and vector phases) holds four query chunks; workgroups
// are persistent, one per CU.
//
// d = 128 (path_fwd_bf16_kernel): every step, the own chunk's too, is taken
// here, with the rank-C carry Q <- Q - (Q W^T) U; a workgroup of 4 waves
// holds two query chunks (32 queries per wave).
//
// Orientation.  All products are formed transposed (S^T = K~ Q^T,
// O^T += V^T P^T, Q^T += (-M^T) Q^T or Q^T -= U^T X^T), so every accumulator
// that feeds a later product (S^T -> P^T, X^T, Q^T) is already in B-operand
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
// Dealing: heaviest query blocks first, and when B*H is a multiple of 8 all
// blocks of one head go to one XCD, so a head's chunks are reused out of that
// XCD's L2.
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

// PV A operands from a V tile kept as it is ([64 tokens][64 d], 16-byte units
// swizzled by swz_v) with LDS transpose loads.  Within each
// group of 16 lanes, ds_read_b64_tr_b16 gives lane i, element t, the element
// i % 4 of the 8 bytes read by lane 4t + i/4.  So lane 4t + q reads 4
// consecutive d of one token, and every lane receives one d column of four
// tokens.  The permutations of the token (k-slot) and d (row) axes act on
// blocks of four, which this access respects.  The operand of k-step ks, rows
// dt, takes two loads (slots 0-3 and 4-7); a lane's 8 byte offsets depend
// on (ks & 1, load, dt), the rows 32 (ks >> 1) further on add 4096 bytes.
//
// One transpose load reads 8 bytes per lane: lanes 0-31 cover 64 bytes of each
// of 4 consecutive token rows, lanes 32-63 the next 4 rows (two 256-byte
// halves; by quarters, 16 lanes cover 32 bytes of each of 4 rows).  The V
// tile's swizzle gv(r) takes row bits 2, 0, 1 as unit bits 0, 1, 2: rows r
// and r + 2 then differ in unit bit 2, so the four rows' pieces of either
// half, or of any quarter, fall on distinct LDS banks (64 banks of 4 bytes
// for a 32-lane half, 32 for a 16-lane quarter).  The swizzle of the other
// tiles, made for 16-byte row reads, puts rows r and r + 2 on the same banks
// here.
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
__device__ __forceinline__ int swz_v(int r) {
    return ((r >> 2) & 1) | ((r & 1) << 1) | (((r >> 1) & 1) << 2);
}
__device__ __forceinline__ void vtr_offsets(unsigned off[8], int lane) {
    const int hh = lane >> 5, hp = (lane >> 4) & 1, j = lane & 15;
#pragma unroll
    for (int par = 0; par < 2; ++par)
#pragma unroll
        for (int ins = 0; ins < 2; ++ins)
#pragma unroll
            for (int dt = 0; dt < 2; ++dt) {
                const int tok = permk(16 * par + 8 * hh + 4 * ins + (j >> 2));
                const int d = permk(32 * dt + 16 * hp + 4 * (j & 3));
                off[(par * 2 + ins) * 2 + dt] =
                    static_cast<unsigned>((tok * 64 + (((d >> 3) ^ swz_v(tok)) << 3) + (d & 7)) * 2);
            }
}
__device__ __forceinline__ bf16x8 pv_operand(const bf16* sv, const unsigned off[8], int dt, int ks) {
    const char* base = reinterpret_cast<const char*>(sv) + 4096 * (ks >> 1);
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(base + off[((ks & 1) * 2 + 0) * 2 + dt]));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(base + off[((ks & 1) * 2 + 1) * 2 + dt]));
    const v4s both[2] = {lo, hi};
    bf16x8 r;
    __builtin_memcpy(&r, both, sizeof(r));
    return r;
}
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

// Asynchronous copy of a [ROWS][COLS] bf16 tile, contiguous in global memory,
// into a swizzled LDS tile.  Each wave instruction fills one contiguous 1 KB
// block of LDS (lane i -> bytes 16i..16i+15); the lane picks the global unit
// that belongs there.
template <int ROWS, int COLS>
__device__ __forceinline__ void copy_async(bf16* lds, const bf16* g, int wave, int lane) {
    constexpr int UPR = COLS / 8;
    constexpr int RPB = 64 / UPR;             // rows per 1 KB block
    constexpr int NBLK = ROWS / RPB;
#pragma unroll
    for (int b = wave; b < NBLK; b += 4) {
        const int r = b * RPB + lane / UPR;
        const int u = (lane % UPR) ^ swz_g<COLS>(r);
        __builtin_amdgcn_global_load_lds((gbl_void*)(g + (size_t)r * COLS + u * 8),
                                         (lds_void*)(lds + b * 512), 16, 0, 0);
    }
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

__device__ __forceinline__ void decode_block(int bid, int BH, int nqb, int& head, int& qb) {
    if ((BH & 7) == 0) {
        const int xcd = bid & 7, j = bid >> 3;
        head = xcd + 8 * (j / nqb);
        qb = nqb - 1 - (j % nqb);
    } else {
        head = bid / nqb;
        qb = nqb - 1 - (bid % nqb);
    }
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

// The running maximum is raised (and O, l rescaled) only when some lane's
// candidate exceeds it by more than this many log2 units, so probabilities
// stay <= 2^kRescaleSlack before the final normalisation.
constexpr float kRescaleSlack = 8.f;

template <int D, bool GATE>
struct WaveState {
    static constexpr int DT = D / 32, KSD = D / 16;
    f32x16 qacc[DT];   // carried query Q^T (fp32); register 8s+t = d 32dt+16s+8hh+t
    bf16x8 qB[KSD];    // its bf16 B operand
    f32x16 oacc[DT];   // O^T (unnormalised), same d mapping
    float m_run, l_run, loc_i;
    double dab;        // gate: sum of chunk sums between the query chunk and the key chunk
    int offD[KSD];     // swizzled offsets of unit 2ks+hh in a D-wide row  (row = 32x + lane%32)
    int offC_[D == 64 ? 1 : 4];   // same in a 64-wide row (d = 64: equal to offD)
    unsigned voff[D == 64 ? 8 : 1]; // d = 64: transpose-load offsets of the PV operands
    __device__ __forceinline__ int offC(int ks) const { return D == 64 ? offD[ks] : offC_[ks]; }
};

template <int D>
struct Stage {
    bf16* k;           // K~  [C][D]
    bf16* w;           // W   [C][D]      (d = 64: the diagonal chunk's, shared)
    bf16* u;           // -U^T [D][C]     (d = 64: the diagonal chunk's, shared)
    bf16* v;           // V^T  [D][C]
    bf16* mt;          // -M^T [D][D]     (d = 64 only)
    float* loc;        // -local log2 gate prefix [C], then the chunk's gate sum
    bf16* gb;          // d = 64 with gate: bias k-step A rows [C][16]
};

// Three-term bf16 split, x = h + m + l to about 24 bits.
__device__ __forceinline__ void split3(float x, bf16& h, bf16& m, bf16& l) {
    h = static_cast<bf16>(x);
    const float r = x - static_cast<float>(h);
    m = static_cast<bf16>(r);
    l = static_cast<bf16>(r - static_cast<float>(m));
}

// One key chunk for one wave.  DIAG: the key chunk is the query's own chunk.
template <int D, bool GATE, bool DIAG>
__device__ __forceinline__ void scan_step(WaveState<D, GATE>& st, const Stage<D>& sg,
                                          const bf16* sY, int l32, int hh, int iloc,
                                          bool carry, float c2) {
    constexpr int C = 64;
    constexpr int DT = D / 32, KSD = D / 16, KSC = C / 16;

    // S^T = K~ Q^T and X^T = W Q^T  (2 tiles of 32 keys).  With the forget
    // gate, one more k-step adds -loc_j / c2 to every logit of key j (the key
    // part of the bias, split into three bf16 terms: a gate that cuts the past
    // makes loc_j of order 1e4, and the cancellation against the query's part
    // must keep fp32 precision), so that c2 * S holds
    // scale*log2(e)*(k~_j . q) + log2 prod f over the key's chunk tail.
    f32x16 s[2], x[2];
#pragma unroll
    for (int kt2 = 0; kt2 < 2; ++kt2) {
#pragma unroll
        for (int v = 0; v < 16; ++v) { s[kt2][v] = 0.f; x[kt2][v] = 0.f; }
        const bf16* ak = sg.k + (32 * kt2 + l32) * D;
        const bf16* aw = sg.w + (32 * kt2 + l32) * D;
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) x[kt2] = mfma32(lds8(aw + st.offD[ks]), st.qB[ks], x[kt2]);
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) s[kt2] = mfma32(lds8(ak + st.offD[ks]), st.qB[ks], s[kt2]);
        if (GATE) {
            bf16 gh, gm, gl;
            split3(-sg.loc[32 * kt2 + l32] * (1.f / c2), gh, gm, gl);
            bf16x8 ag = {};
            bf16x8 ones = {};
            if (hh == 0) {
                ag[0] = gh;
                ag[1] = gm;
                ag[2] = gl;
                ones[0] = static_cast<bf16>(1.f);
                ones[1] = static_cast<bf16>(1.f);
                ones[2] = static_cast<bf16>(1.f);
            }
            s[kt2] = mfma32(ag, ones, s[kt2]);
        }
    }
    if (DIAG) {
        // S^T += Y^T strictUpper(X)^T ;  X^T <- lower part (m <= i)
        bf16x8 xu[KSC];
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks)
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int v = 8 * (ks & 1) + t;
                const int m = 32 * (ks >> 1) + 8 * (v >> 2) + 4 * hh + (v & 3);
                const float xv = x[ks >> 1][v];
                xu[ks][t] = static_cast<bf16>(m > iloc ? xv : 0.f);
                x[ks >> 1][v] = (m <= iloc) ? xv : 0.f;
            }
#pragma unroll
        for (int kt2 = 0; kt2 < 2; ++kt2) {
            const bf16* ay = sY + (32 * kt2 + l32) * C;
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) s[kt2] = mfma32(lds8(ay + st.offC(ks)), xu[ks], s[kt2]);
        }
    }
    // carry the query through this chunk:  Q^T += (-U^T) X^T   (independent of
    // the softmax below, so its MFMAs overlap with the vector work)
    if (carry) {
        bf16x8 xB[KSC];
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) xB[ks] = pack8(x[ks >> 1], ks & 1);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const bf16* au = sg.u + (32 * dt + l32) * C;
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) st.qacc[dt] = mfma32(lds8(au + st.offC(ks)), xB[ks], st.qacc[dt]);
        }
    }

    // online softmax in log2 units: z = c2 * S + a_i.  Lane holds keys
    // j = 32*kt2 + 8*(v/4) + 4*hh + v%4 of query iloc; lane^32 holds the rest.
    const float a_i = GATE ? st.loc_i + static_cast<float>(st.dab) : 0.f;
    float mx = -INFINITY;
#pragma unroll
    for (int kt2 = 0; kt2 < 2; ++kt2)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            if (DIAG && (32 * kt2 + 8 * (v >> 2) + 4 * hh + (v & 3)) > iloc) s[kt2][v] = -INFINITY;
            mx = fmaxf(mx, s[kt2][v]);
        }
    mx = pair_max(mx);
    const float cand = fmaf(mx, c2, a_i);
    if (__any(cand > st.m_run + kRescaleSlack)) {
        const float m_new = fmaxf(st.m_run, cand);
        const float alpha = fast_exp2(st.m_run - m_new);
        st.m_run = m_new;
        st.l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int v = 0; v < 16; ++v) st.oacc[dt][v] *= alpha;
    }
    const float msub = st.m_run - a_i;
    bf16x8 pB[KSC];
    float psum = 0.f;
#pragma unroll
    for (int ks = 0; ks < KSC; ++ks) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
            pB[ks][t] = static_cast<bf16>(fast_exp2(fmaf(s[ks >> 1][8 * (ks & 1) + t], c2, -msub)));
        // row sum of the rounded probabilities (the values the PV product uses)
#pragma unroll
        for (int t = 0; t < 8; t += 2) {
            const bf16x2 pr = {pB[ks][t], pB[ks][t + 1]};
            psum = __builtin_amdgcn_fdot2_f32_bf16(pr, bf16x2{bf16(1.f), bf16(1.f)}, psum, false);
        }
    }
    st.l_run += psum;

    // O^T += V^T P^T (d = 64: V as it is, through transpose loads)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        const bf16* av = sg.v + (32 * dt + l32) * C;
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) {
            bf16x8 a8;
            if constexpr (D == 64) a8 = pv_operand(sg.v, st.voff, dt, ks);
            else a8 = lds8(av + st.offC(ks));
            st.oacc[dt] = mfma32(a8, pB[ks], st.oacc[dt]);
        }
    }
    if (carry) {
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) st.qB[ks] = pack8(st.qacc[ks >> 1], ks & 1);
    }
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
template <bool GATE>
__device__ __forceinline__ void raise_max(WaveState<64, GATE>& st, float shift) {
    const float alpha = fast_exp2(-shift);
    st.m_run += shift;
    st.l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) st.oacc[dt][v] *= alpha;
}

// Per-lane setup shared by both kernels: block decode, query load, state.
template <int D, bool GATE>
struct ScanSetup {
    int head, qb, qc, iloc, qi;
    bool active, qvalid;
};

// The wave's query chunk is qc, its query row within that chunk iloc.
template <int D, bool GATE>
__device__ __forceinline__ ScanSetup<D, GATE> scan_setup(const FwdArgs& a, WaveState<D, GATE>& st, int head,
                                                          int qb, int qc, int iloc, int l32, int hh) {
    constexpr int C = 64, DT = D / 32, KSD = D / 16;
    ScanSetup<D, GATE> u;
    u.head = head;
    u.qb = qb;
    u.qc = qc;
    u.active = u.qc < a.N;
    u.iloc = iloc;
    u.qi = u.qc * C + u.iloc;
    u.qvalid = u.active && u.qi < a.L;
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) st.offD[ks] = ((2 * ks + hh) ^ swz_g<D>(l32)) << 3;
    if (D != 64) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) st.offC_[ks & (D == 64 ? 0 : 3)] = ((2 * ks + hh) ^ swz_g<C>(l32)) << 3;
    }
    const bf16* qrow = static_cast<const bf16*>(a.q) + ((size_t)u.head * a.L + (u.qvalid ? u.qi : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
        bf16x8 q8 = {};
        if (u.qvalid) q8 = lds8(qrow + 16 * ks + 8 * hh);
        st.qB[ks] = q8;
#pragma unroll
        for (int t = 0; t < 8; ++t) st.qacc[ks >> 1][8 * (ks & 1) + t] = static_cast<float>(q8[t]);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) st.oacc[dt][v] = 0.f;
    st.m_run = -INFINITY;
    st.l_run = 0.f;
    st.loc_i = (GATE && u.qvalid) ? a.loc[(size_t)u.head * a.N * C + u.qi] : 0.f;
    st.dab = 0.0;
    return u;
}

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

// d = 128: every key chunk carries the query with the rank-C form
// Q <- Q - (Q W^T) U.
template <int D, bool GATE>
__global__ __launch_bounds__(256, 1) void path_fwd_bf16_kernel(const FwdArgs a) {
    constexpr int C = 64;
    constexpr int TILE = C * D;   // elements of every staged tile

    // two stage sets (distinct objects so the DMA target and the tiles being
    // read are known not to alias), the diagonal-chunk Y^T tile, gate terms
    __shared__ __attribute__((aligned(1024))) bf16 sK0[TILE];
    __shared__ __attribute__((aligned(1024))) bf16 sW0[TILE];
    __shared__ __attribute__((aligned(1024))) bf16 sU0[TILE];
    __shared__ __attribute__((aligned(1024))) bf16 sV0[TILE];
    __shared__ __attribute__((aligned(1024))) bf16 sK1[TILE];
    __shared__ __attribute__((aligned(1024))) bf16 sW1[TILE];
    __shared__ __attribute__((aligned(1024))) bf16 sU1[TILE];
    __shared__ __attribute__((aligned(1024))) bf16 sV1[TILE];
    __shared__ __attribute__((aligned(1024))) bf16 sY[C * C];
    __shared__ __attribute__((aligned(256))) float sLoc0[C];
    __shared__ __attribute__((aligned(256))) float sLoc1[C];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int L = a.L, N = a.N, Lp = N * C;
    WaveState<D, GATE> st;
    int head0, qb0;
    decode_block(blockIdx.x, a.BH, a.nqb, head0, qb0);
    const ScanSetup<D, GATE> u =
        scan_setup<D, GATE>(a, st, head0, qb0, 2 * qb0 + (wave >> 1), (wave & 1) * 32 + l32, l32, hh);
    const int head = u.head, qb = u.qb, qc = u.qc, iloc = u.iloc;
    const bool active = u.active;

    const bf16* kt = static_cast<const bf16*>(a.kt) + (size_t)head * Lp * D;
    const bf16* win = static_cast<const bf16*>(a.w) + (size_t)head * L * D;
    const bf16* ut = static_cast<const bf16*>(a.ut) + (size_t)head * N * D * C;
    const bf16* vt = static_cast<const bf16*>(a.vt) + (size_t)head * N * D * C;
    const bf16* yt = static_cast<const bf16*>(a.yt) + (size_t)head * N * C * C;
    const float* locg = GATE ? a.loc + (size_t)head * Lp : nullptr;

    const Stage<D> stage0{sK0, sW0, sU0, sV0, nullptr, sLoc0, nullptr};
    const Stage<D> stage1{sK1, sW1, sU1, sV1, nullptr, sLoc1, nullptr};

    auto issue = [&](const Stage<D>& sg, int kc) {     // full chunk, asynchronous
        copy_async<C, D>(sg.k, kt + (size_t)kc * C * D, wave, lane);
        copy_async<C, D>(sg.w, win + (size_t)kc * C * D, wave, lane);
        copy_async<D, C>(sg.u, ut + (size_t)kc * D * C, wave, lane);
        copy_async<D, C>(sg.v, vt + (size_t)kc * D * C, wave, lane);
        if (GATE && wave == 0)
            __builtin_amdgcn_global_load_lds((gbl_void*)(locg + kc * C + lane),
                                             (lds_void*)sg.loc, 4, 0, 0);
    };
    const float c2 = a.scale2;

    // prologue: the top chunk (possibly the ragged last one: its W rows past
    // L are zero-filled) and its Y^T
    int kc = min(2 * qb + 1, N - 1);
    copy_async<C, D>(sK0, kt + (size_t)kc * C * D, wave, lane);
    copy_guarded<C, D>(sW0, win + (size_t)kc * C * D, min(C, L - kc * C), tid);
    copy_async<D, C>(sU0, ut + (size_t)kc * D * C, wave, lane);
    copy_async<D, C>(sV0, vt + (size_t)kc * D * C, wave, lane);
    if (GATE && wave == 0)
        __builtin_amdgcn_global_load_lds((gbl_void*)(locg + kc * C + lane), (lds_void*)sLoc0, 4, 0, 0);
    copy_async<C, C>(sY, yt + (size_t)kc * C * C, wave, lane);
    wait_vmem();
    __syncthreads();

    auto compute = [&](const Stage<D>& sg, int kcur) {
        if (!active || kcur > qc) return;
        const bool carry = kcur > 0;
        if (kcur == qc)
            scan_step<D, GATE, true>(st, sg, sY, l32, hh, iloc, carry, c2);
        else
            scan_step<D, GATE, false>(st, sg, sY, l32, hh, iloc, carry, c2);
        if (GATE && carry) st.dab += static_cast<double>(a.csum[(size_t)head * N + kcur]);
    };

    for (;;) {
        if (kc > 0) issue(stage1, kc - 1);
        compute(stage0, kc);
        wait_vmem();
        __syncthreads();
        if (kc == 0) break;
        --kc;
        if (kc >= 2 * qb) {           // second diagonal chunk of this block
            copy_async<C, C>(sY, yt + (size_t)kc * C * C, wave, lane);
            wait_vmem();
            __syncthreads();
        }
        if (kc > 0) issue(stage0, kc - 1);
        compute(stage1, kc);
        wait_vmem();
        __syncthreads();
        if (kc == 0) break;
        --kc;
    }
    scan_store<D, GATE>(a, st, u, hh);
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
// k % 2 and are copied two phases before their first use.
// ---------------------------------------------------------------------------

// Matrix phase of one wave: O^T += V^T P^T for the pending probabilities pB
// (V tile sv), then with QK the logits of the staged chunk sg (left in s as
// z - m_run), and the -M^T operands of the chunk's carry read into opm (the
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
// Q^T += (-M^T) Q^T (operands opm from the matrix phase; the MFMAs go first
// and run under the probabilities), the logits s turned into probabilities
// pB (raising the running maximum when a row sum passes kRescaleTrigger),
// and the carried query's new operand.
template <bool GATE>
__device__ __forceinline__ void pp_vphase(WaveState<64, GATE>& st, const f32x16 s[2], bf16x8 pB[4],
                                          const bf16x8 opm[8]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) st.qacc[dt] = mfma32(opm[4 * dt + ks], st.qB[ks], st.qacc[dt]);
    float psum = tile_probs(s[0], pB[0], pB[1], 0.f) + tile_probs(s[1], pB[2], pB[3], 0.f);
    if (__any(!(psum <= kRescaleTrigger))) {
        const float shift = fmaxf(pair_max(fmaxf(tile_max(s[0]), tile_max(s[1]))), 0.f);
        raise_max(st, shift);
        psum = tile_probs(s[0], pB[0], pB[1], shift) + tile_probs(s[1], pB[2], pB[3], shift);
    }
    st.l_run += psum;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) st.qB[ks] = pack8(st.qacc[ks >> 1], ks & 1);
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
    __shared__ __attribute__((aligned(1024))) ChunkTiles km0;
    __shared__ __attribute__((aligned(1024))) ChunkTiles km1;

    const int wave_u = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const bool leader = wave_u >= 4;
    const int nqb = (a.N + 3) / 4;

    // One query block (head, qb): query chunks 4qb .. 4qb+3 of one head.  The
    // arguments and the lane id come in through opaque copies, so that
    // nothing derived from them is kept live from one block to the next.
    auto item = [&](const int head, const int qb, const FwdArgs& a, const int lane_in) {
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
    {
        // the state after the query's own chunk, from the prepare stage: the
        // query carried to its chunk start (scaled by scale*log2(e)), the
        // pending probabilities of its own keys, their maximum and sum
        const size_t row = (size_t)head * Lp + (active ? u.qi : 0);
        const bf16* qrow = static_cast<const bf16*>(a.qt) + row * D;
        const bf16* prow = static_cast<const bf16*>(a.pd) + row * C;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            st.offD[ks] = ((2 * ks + hh) ^ swz_g<D>(l32)) << 3;
            st.qB[ks] = lds8(qrow + 16 * ks + 8 * hh);
            pB[ks] = lds8(prow + 16 * ks + 8 * hh);
#pragma unroll
            for (int t = 0; t < 8; ++t) st.qacc[ks >> 1][8 * (ks & 1) + t] = static_cast<float>(st.qB[ks][t]);
        }
        const f32x2 ml = *reinterpret_cast<const f32x2*>(a.ml + 2 * row);
        st.m_run = ml[0];
        st.l_run = hh == 0 ? ml[1] : 0.f;   // the two lane halves' sums are added at the end
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
            for (int v = 0; v < 16; ++v) st.oacc[dt][v] = 0.f;
        st.loc_i = GATE ? a.loc[row] : 0.f;
        st.dab = GATE ? static_cast<double>(a.csum[(size_t)head * N + (active ? qc : 0)]) : 0.0;
    }
    vtr_offsets(st.voff, lane);

    const bf16* kt = static_cast<const bf16*>(a.kt) + (size_t)head * Lp * D;
    const bf16* vin = static_cast<const bf16*>(a.v) + (size_t)head * L * D;
    const bf16* mtg = static_cast<const bf16*>(a.mt) + (size_t)head * N * D * D;
    const float* locg = GATE ? a.loc + (size_t)head * Lp : nullptr;
    const float* csg = GATE ? a.csum + (size_t)head * N : nullptr;
    const bf16* gbg = GATE ? static_cast<const bf16*>(a.gb) + (size_t)head * Lp * 16 : nullptr;

    const Stage<D> set0{km0.k, nullptr, nullptr, km0.v, km0.m, km0.loc, km0.gb};
    const Stage<D> set1{km1.k, nullptr, nullptr, km1.v, km1.m, km1.loc, km1.gb};

    // every [64][64] tile: wave w copies its 1 KB block w (rows 8w .. 8w+7)
    auto tile = [&](bf16* lds, const bf16* g) {
        __builtin_amdgcn_global_load_lds((gbl_void*)(reinterpret_cast<const char*>(g) + loff),
                                         (lds_void*)(reinterpret_cast<char*>(lds) + wave_u * 1024), 16, 0, 0);
    };
    auto issue_km = [&](const Stage<D>& sg, int kc) {   // K~, -M^T, bias rows, gate terms
        tile(sg.k, kt + (size_t)kc * TILE);
        tile(sg.mt, mtg + (size_t)kc * TILE);
        if (GATE && wave_u < 2)
            __builtin_amdgcn_global_load_lds((gbl_void*)(gbg + (size_t)kc * C * 16 + wave_u * 512 + lane * 8),
                                             (lds_void*)(sg.gb + wave_u * 512), 16, 0, 0);
        if (GATE && wave_u == 2) {
            __builtin_amdgcn_global_load_lds((gbl_void*)(locg + kc * C + lane), (lds_void*)sg.loc, 4, 0, 0);
            if (lane == 0)
                __builtin_amdgcn_global_load_lds((gbl_void*)(csg + kc), (lds_void*)(sg.loc + C), 4, 0, 0);
        }
    };
    auto issue_v = [&](const Stage<D>& sg, int kc) {
        if ((kc + 1) * C <= L)
            __builtin_amdgcn_global_load_lds(
                (gbl_void*)(reinterpret_cast<const char*>(vin + (size_t)kc * TILE) + vloff),
                (lds_void*)(reinterpret_cast<char*>(sg.v) + wave_u * 1024), 16, 0, 0);
        else
            copy_guarded<C, D, NT, true>(sg.v, vin + (size_t)kc * TILE, L - kc * C, tid);   // ragged: zero rows
    };

    // ---- key chunks ktop-1 .. 0 in phases; ktop = the block's top chunk.
    // Chunk k's K~/-M^T/gate terms sit in set k % 2, its V tile in that set's
    // V tile.  A wave works on chunk k only when k < qc (its own chunk was
    // done by the prepare stage, whose probabilities are pending against
    // V(qc)); the other waves of the block keep the copies and barriers.
    // Every wave runs
    //     for k = ktop-1 .. 0:  M(k); barrier; V(k); barrier        then PV(0)
    // where M(k) = PV(k+1), logits and carry of k, and V(k) = the
    // probabilities of k.  The followers (waves 0..3) enter one barrier late,
    // so between two barriers one wave of each SIMD is in a matrix phase and
    // the other in a vector phase.  Copies: at the start of its M(k) a leader
    // issues its blocks of chunk k-1 (K~/-M^T) and V(k); at the start of its
    // V(k) a follower issues its blocks of chunk k-2 and V(k-1) -- the same
    // moment, one phase after the buffers' last reads.  Leaders wait for their
    // copies at the end of V(k), followers at the end of M(k): two phases
    // later, and before the barrier that opens the first phase reading them.
    // The prologue stages V(ktop), and chunk ktop-1 with V(ktop-1), whole. ----
    const int ktop = min(4 * qb + 3, N - 1);
    if (ktop & 1) {
        issue_v(set1, ktop);
        issue_km(set0, ktop - 1);
        issue_v(set0, ktop - 1);
    } else {
        issue_v(set0, ktop);
        if (ktop >= 1) {
            issue_km(set1, ktop - 1);
            issue_v(set1, ktop - 1);
        }
    }
    wait_vmem();
    __syncthreads();
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
            phase_barrier();
        }
        auto iter = [&](int k, const Stage<D>& ck, const Stage<D>& cn) {
            // ck: chunk k and V(k); cn: chunk k +- 1 and V(k +- 1).  Chunks
            // below ktop are full, so V is copied without a guard.
            if (leader) {
                if (k >= 1) kissue(cn, k - 1);
                if (k < ktop - 1) dma_lds16(vin + (size_t)k * TILE, vloff, ck.v + wave_u * 512);
            }
            const bool go = active && k < qc;
            if (go) pp_mphase<GATE, true>(st, s, pB, opm, ck, cn.v, l32, hh);
            if (!leader) wait_vmem();
            phase_barrier();
            if (!leader) {
                if (k >= 2) kissue(ck, k - 2);
                if (k >= 1) dma_lds16(vin + (size_t)(k - 1) * TILE, vloff, cn.v + wave_u * 512);
            }
            if (go) pp_vphase<GATE>(st, s, pB, opm);
            if (leader) wait_vmem();
            phase_barrier();
        };
        int k = ktop - 1;
        if ((k & 1) == 0) {           // k even: one step to reach the odd/even pairs
            iter(k, set0, set1);
            --k;
        }
        for (; k >= 0; k -= 2) {     // k odd, then k - 1 even
            iter(k, set1, set0);
            iter(k - 1, set0, set1);
        }
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
    for (int t = 0;; ++t) {                      // t-th block of this workgroup: pair r + R (t / 2), heavy half first
        int i, qb;
        if (single) {                            // block r of this workgroup's heads, heaviest first
            if (t > 0) break;
            i = r / nqb;
            qb = nqb - 1 - r % nqb;
        } else {
            const int j = r + R * (t >> 1);
            if (j >= npairs) break;
            const int pr = j % P;
            i = j / P;
            qb = (t & 1) ? pr : nqb - 1 - pr;
            if ((t & 1) && qb == nqb - 1 - pr) continue;   // the lone middle block of an odd nqb
        }
        __syncthreads();                         // the previous block's tiles are no longer read
        typedef const __attribute__((address_space(4))) FwdArgs* ArgPtr;
        ArgPtr ap = (ArgPtr)__builtin_amdgcn_kernarg_segment_ptr();
        int ln = static_cast<int>(threadIdx.x & 63);
        asm volatile("" : "+s"(ap), "+v"(ln));
        item(by_xcd ? xcd + 8 * i : i, qb, *(const FwdArgs*)ap, ln);
    }
}

hipError_t launch_path_fwd_bf16(const FwdArgs& args, bool gate, hipStream_t s) {
    FwdArgs a = args;
    const dim3 grid(a.BH * a.nqb), block(256);
    if (a.D == 64) {
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
        if (gate) hipLaunchKernelGGL((path_fwd_bf16_d64pp_kernel<true>), gridp, block8, 0, s, a);
        else hipLaunchKernelGGL((path_fwd_bf16_d64pp_kernel<false>), gridp, block8, 0, s, a);
    } else if (a.D == 128) {
        if (gate) hipLaunchKernelGGL((path_fwd_bf16_kernel<128, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((path_fwd_bf16_kernel<128, false>), grid, block, 0, s, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace path
