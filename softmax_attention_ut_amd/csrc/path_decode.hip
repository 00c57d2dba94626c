// path_decode: one PaTH decode step with the in-place key-cache update
// (gfx950).
//
// At step t every cached key is multiplied by the new transition,
//     k_j <- (I - beta_t w_t w_t^T) k_j          (j < t),
// the new key and value are stored at slot t, and q_t attends over slots
// 0..t with plain softmax (Dutch summary section 3, "Inferentie"; Chinese
// notes, inference paragraph: decoding then reduces to standard softmax
// decoding).  The update, the write-back and the score are one pass over
// the cache: per key, w.k and q.k are reduced together, the updated key is
// stored, and the score is q.k - beta (w.k)(q.w).
//
// Split-sequence layout: block (split, head) owns a run of consecutive slots
// (a multiple of 64, sized so that every block of the step is resident at
// once) and writes a partial (m, l, o) in log2 units; path_decode_combine
// merges the splits of a head.  Each group of G = D/8 lanes owns one key (16 bytes per
// lane), so a wave streams 64/G keys per pass with 16-byte accesses.
#include "path_internal.h"

#include <atomic>

namespace path {

template <int D, bool GATE, bool PAGED>
__global__ __launch_bounds__(256) void path_decode_split_kernel(const DecodeArgs a) {
    constexpr int G = D / 8;              // lanes per key
    constexpr int KPW = 64 / G;           // keys per wave pass
    constexpr int KPB = 4 * KPW;          // keys per block pass
    __shared__ float sPart[4 * KPW][D + 2];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane / G, gl = lane % G;
    const int split = blockIdx.x, head = blockIdx.y;
    const int t = a.t;
    const int j0 = split * a.keys_per_split;
    const int j1 = min(j0 + a.keys_per_split, t + 1);

    const bf16* qh = static_cast<const bf16*>(a.q) + (size_t)head * D;
    const bf16* wh = static_cast<const bf16*>(a.w) + (size_t)head * D;
    const bf16* kh = static_cast<const bf16*>(a.k) + (size_t)head * D;
    const bf16* vh = static_cast<const bf16*>(a.v) + (size_t)head * D;
    // contiguous: rows head * T_max + j.  Paged: a pass of 2 KPB keys never
    // crosses a 64-key boundary and pages are multiples of 64 keys, so the
    // whole pass is in one page, looked up once per pass (a uniform load).
    bf16* const kbase = static_cast<bf16*>(a.k_cache);
    bf16* const vbase = static_cast<bf16*>(a.v_cache);
    long long rb = (long long)head * a.T_max;     // cache row of slot j: rb + j
    const float beta = a.beta[head];
    // forget gate (PaTH-FoX): the logit of key j gains F_t - F_j (natural
    // log, F = inclusive prefix sum of log f), taken to log2 units.  F_t is
    // formed from the cached F_{t-1}; the first split appends it to the cache.
    const float* fc = GATE ? a.f_cache + (size_t)head * a.T_max : nullptr;
    float f_t = 0.f;
    if (GATE) {
        f_t = (t > 0 ? fc[t - 1] : 0.f) + a.log_f[head];
        if (split == 0 && tid == 0) a.f_cache[(size_t)head * a.T_max + t] = f_t;
    }

    float qf[8], wf[8];
    {
        const bf16x8 q8 = *reinterpret_cast<const bf16x8*>(qh + 8 * gl);
        const bf16x8 w8 = *reinterpret_cast<const bf16x8*>(wh + 8 * gl);
#pragma unroll
        for (int e = 0; e < 8; ++e) { qf[e] = static_cast<float>(q8[e]); wf[e] = static_cast<float>(w8[e]); }
    }
    float qw = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) qw += qf[e] * wf[e];
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) qw += __shfl_xor(qw, off, G);

    float m = -INFINITY, l = 0.f, o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;

    // Two keys per lane group per pass (the second KPB keys after the
    // first), their loads issued together so that each wave has two lines
    // of K and of V in flight.
    for (int jb = j0; jb < j1; jb += 2 * KPB) {
        if (PAGED) {
            // rows of this pass: (page * H + h) * P + (j % P) = r + (j - jb)
            const long long r = cache_row(a.map, head, jb);
            if (r < 0) continue;          // a page outside the pool: left out
            rb = r - jb;
        }
        int jj[2];
        bool ok[2];
        bf16x8 k8[2], v8[2];
        float fj[2] = {0.f, 0.f};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            jj[h] = jb + h * KPB + wave * KPW + g;
            ok[h] = jj[h] < j1;
            k8[h] = v8[h] = bf16x8{};
            if (ok[h]) {
                k8[h] = (jj[h] < t) ? *reinterpret_cast<const bf16x8*>(kbase + (rb + jj[h]) * D + 8 * gl)
                                    : *reinterpret_cast<const bf16x8*>(kh + 8 * gl);
                v8[h] = (jj[h] < t) ? *reinterpret_cast<const bf16x8*>(vbase + (rb + jj[h]) * D + 8 * gl)
                                    : *reinterpret_cast<const bf16x8*>(vh + 8 * gl);
                if (GATE) fj[h] = (jj[h] < t) ? fc[jj[h]] : f_t;
            }
        }
        float s[2], pw[2], pq[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            pw[h] = 0.f;
            pq[h] = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float kf = static_cast<float>(k8[h][e]);
                pw[h] += wf[e] * kf;
                pq[h] += qf[e] * kf;
            }
        }
#pragma unroll
        for (int off = G / 2; off > 0; off >>= 1) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                pw[h] += __shfl_xor(pw[h], off, G);
                pq[h] += __shfl_xor(pq[h], off, G);
            }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            s[h] = -INFINITY;
            if (!ok[h]) continue;
            if (jj[h] < t) {
                const float ba = beta * pw[h];
                bf16x8 k8n;
#pragma unroll
                for (int e = 0; e < 8; ++e) k8n[e] = static_cast<bf16>(static_cast<float>(k8[h][e]) - ba * wf[e]);
                *reinterpret_cast<bf16x8*>(kbase + (rb + jj[h]) * D + 8 * gl) = k8n;
                s[h] = (pq[h] - ba * qw) * a.scale2;
            } else {   // j == t: the new key and value enter unchanged
                *reinterpret_cast<bf16x8*>(kbase + (rb + jj[h]) * D + 8 * gl) = k8[h];
                *reinterpret_cast<bf16x8*>(vbase + (rb + jj[h]) * D + 8 * gl) = v8[h];
                s[h] = pq[h] * a.scale2;
            }
            if (GATE) s[h] += (f_t - fj[h]) * kLog2e;
        }
        if (ok[0]) {   // ok[1] implies ok[0]
            const float mn = fmaxf(m, fmaxf(s[0], s[1]));
            const float sc = exp2f(m - mn);
            const float p0 = exp2f(s[0] - mn);
            const float p1 = ok[1] ? exp2f(s[1] - mn) : 0.f;
            l = l * sc + p0 + p1;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                o[e] = o[e] * sc + p0 * static_cast<float>(v8[0][e]) + p1 * static_cast<float>(v8[1][e]);
            m = mn;
        }
    }
    // merge the 4*KPW key groups of the block
    const int grp = wave * KPW + g;
#pragma unroll
    for (int e = 0; e < 8; ++e) sPart[grp][8 * gl + e] = o[e];
    if (gl == 0) { sPart[grp][D] = m; sPart[grp][D + 1] = l; }
    __syncthreads();
    if (tid < D) {
        float mm = -INFINITY;
        for (int r = 0; r < 4 * KPW; ++r) mm = fmaxf(mm, sPart[r][D]);
        float ll = 0.f, oo = 0.f;
        for (int r = 0; r < 4 * KPW; ++r) {
            const float mr = sPart[r][D];
            if (mr == -INFINITY) continue;
            const float sc = exp2f(mr - mm);
            ll += sPart[r][D + 1] * sc;
            oo += sPart[r][tid] * sc;
        }
        float* part = a.part + ((size_t)head * a.nsplit + split) * (D + 2);
        part[tid] = oo;
        if (tid == 0) { part[D] = mm; part[D + 1] = ll; }
    }
}

template <int D>
__global__ __launch_bounds__(256) void path_decode_combine_kernel(const DecodeArgs a) {
    // One workgroup per head.  The head's partials (contiguous, nsplit rows
    // of D + 2 floats) are read into LDS in one coalesced round per group of
    // up to SG splits; thread e < D then folds the group into its running
    // (m, l, o_e): group maximum from LDS, weights exp2(m_s - m).
    constexpr int SG = 48;                // splits per LDS group (25 KB at D = 128)
    __shared__ float sp[SG * (D + 2)];
    const int head = blockIdx.x, tid = threadIdx.x;
    const int ns = a.nsplit;
    const float* part = a.part + (size_t)head * ns * (D + 2);
    float m = -INFINITY, l = 0.f, o = 0.f;
    for (int s0 = 0; s0 < ns; s0 += SG) {
        const int n = min(SG, ns - s0);
        const float* src = part + (size_t)s0 * (D + 2);
        if (s0 > 0) __syncthreads();      // the previous group is no longer read
        for (int i = tid; i < n * (D + 2); i += 256) sp[i] = src[i];
        __syncthreads();
        if (tid < D) {
            float mg = m;
            for (int sIdx = 0; sIdx < n; ++sIdx) mg = fmaxf(mg, sp[sIdx * (D + 2) + D]);
            if (mg != -INFINITY) {
                const float c = exp2f(m - mg);
                l *= c;
                o *= c;
                for (int sIdx = 0; sIdx < n; ++sIdx) {
                    const float ms = sp[sIdx * (D + 2) + D];
                    if (ms == -INFINITY) continue;
                    const float wgt = exp2f(ms - mg);
                    l += sp[sIdx * (D + 2) + D + 1] * wgt;
                    o += sp[sIdx * (D + 2) + tid] * wgt;
                }
                m = mg;
            }
        }
    }
    if (tid < D) {
        static_cast<bf16*>(a.out)[(size_t)head * D + tid] = static_cast<bf16>(o / l);
        if (tid == 0 && a.lse) a.lse[head] = (m + log2f(l)) * kLn2;
    }
}

// Workgroups of the split kernel that fit on the current device at once
// (its CU count times the kernel's occupancy), queried once per device and d
// and kept in a process-wide cache (atomic: concurrent first calls may both
// query and store the same value).
static hipError_t resident_split_blocks(int D, int& n) {
    static std::atomic<int> cache[64][2];
    int dev = 0, ncu = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::atomic<int>* slot = (dev >= 0 && dev < 64) ? &cache[dev][D == 128] : nullptr;
    if (slot) {
        const int v = slot->load(std::memory_order_relaxed);
        if (v > 0) {
            n = v;
            return hipSuccess;
        }
    }
    e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = D == 64 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, path_decode_split_kernel<64, true, true>, 256, 0)
                : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, path_decode_split_kernel<128, true, true>, 256, 0);
    if (e != hipSuccess) return e;
    n = ncu * (per_cu > 0 ? per_cu : 1);
    if (slot) slot->store(n, std::memory_order_relaxed);
    return hipSuccess;
}

// Split partials of path_decode_step_noalloc, for callers that cannot
// allocate: one array per device, held until the process ends.  Host code
// never passes the array's name to a kernel (on the host it names a host-side
// stand-in); it passes the device address from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
    static std::atomic<void*> addr[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    void* p = addr[dev].load(std::memory_order_acquire);
    if (!p) {       // first call on this device (concurrent first calls store the same value)
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

hipError_t launch_path_decode(const DecodeArgs& args, int D, hipStream_t s) {
    if (D != 64 && D != 128) return hipErrorInvalidValue;
    // Split the t + 1 keys of each head so that all (split, head) workgroups
    // run in one round: a second, partly filled round would leave most CUs
    // idle for its whole length.  Splits are multiples of 64 keys (whole
    // passes of a workgroup), at most ceil(T_max / 64) of them.
    int resident = 0;
    hipError_t e = resident_split_blocks(D, resident);
    if (e != hipSuccess) return e;
    DecodeArgs a = args;
    const int nkeys = a.t + 1;
    const int want = (resident + a.BH - 1) / a.BH;               // splits per head
    int kps = (nkeys + want - 1) / want;
    kps = ((kps + kDecodeSplitQuantum - 1) / kDecodeSplitQuantum) * kDecodeSplitQuantum;
    a.keys_per_split = kps;
    a.nsplit = (nkeys + kps - 1) / kps;
    const dim3 grid(a.nsplit, a.BH), block(256);
    const bool gate = a.f_cache != nullptr, paged = a.map.table != nullptr;
#define PATH_SPLIT(DD, GG, PP) hipLaunchKernelGGL((path_decode_split_kernel<DD, GG, PP>), grid, block, 0, s, a)
    if (D == 64) {
        if (paged) { if (gate) PATH_SPLIT(64, true, true); else PATH_SPLIT(64, false, true); }
        else { if (gate) PATH_SPLIT(64, true, false); else PATH_SPLIT(64, false, false); }
        hipLaunchKernelGGL(path_decode_combine_kernel<64>, dim3(a.BH), dim3(256), 0, s, a);
    } else {
        if (paged) { if (gate) PATH_SPLIT(128, true, true); else PATH_SPLIT(128, false, true); }
        else { if (gate) PATH_SPLIT(128, true, false); else PATH_SPLIT(128, false, false); }
        hipLaunchKernelGGL(path_decode_combine_kernel<128>, dim3(a.BH), dim3(256), 0, s, a);
    }
#undef PATH_SPLIT
    return hipGetLastError();
}

// Gate cache of a FoX prefill: F_j = sum_{s <= j} log f_s for j < L, one
// workgroup per head.  Each thread sums a contiguous run of L / 256 tokens
// in fp64, the runs' totals are scanned across the workgroup, and each
// thread then writes its run's prefix sums (rounded to fp32).
__global__ __launch_bounds__(256) void path_fcache_kernel(const FcacheArgs a) {
    __shared__ double sTot[256];
    const int head = blockIdx.x, tid = threadIdx.x;
    const int run = (a.L + 255) / 256;
    const int r0 = min(tid * run, a.L), r1 = min(r0 + run, a.L);
    const float* lf = a.log_f + (size_t)head * a.L;
    double tot = 0.0;
    for (int j = r0; j < r1; ++j) tot += static_cast<double>(lf[j]);
    sTot[tid] = tot;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {     // inclusive scan of the run totals
        const double y = tid >= off ? sTot[tid - off] : 0.0;
        __syncthreads();
        sTot[tid] += y;
        __syncthreads();
    }
    double acc = sTot[tid] - tot;                 // sum before this run
    float* fc = a.f_cache + (size_t)head * a.T_max;
    for (int j = r0; j < r1; ++j) {
        acc += static_cast<double>(lf[j]);
        fc[j] = static_cast<float>(acc);
    }
}

hipError_t launch_path_fcache(const FcacheArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(path_fcache_kernel, dim3(a.BH), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace path
