// kvc_schedule.h -- persistent, position-balanced work split for the decode
// kernels ("stream" mode).
//
// The attention of one (sequence b, KV head j) unit over positions [0, L_b)
// may be cut anywhere: partial results over disjoint position ranges combine
// exactly by log-sum-exp ("KV Cache 优化与注意力机制加速" (plumephp.com)
// sections 2.2-2.5: online-softmax rescaling and splitting the sequence
// dimension).  Stream mode lays all units end to end -- unit u = b*g + j
// occupies global positions [U_u, U_u + L_b) with U_u = g*cum[b] + j*L_b,
// cum[b] = L_0 + ... + L_{b-1} -- and gives work-group p of P the range
// [start(p), start(p+1)), start(p) = floor(p * total / P).  Every work-group
// streams the same number of positions whatever the length mix.
//
// Within its range a work-group visits one segment per unit it touches.  A
// segment that covers its whole unit writes the final rows; otherwise it
// writes a partial record (normalised O and base-2 lse) into slot k of the
// work-group: k = 0 for its first segment, 1 for its last.  Only the first
// and the last segment of a range can be partial.  A separate merge pass
// combines the partial records of every unit that spans several
// work-groups, and writes the rows of length-0 sequences.
#pragma once

#include "kvc_device.h"

namespace kvc {

__device__ __forceinline__ long long stream_start(long long p, long long total, long long P) {
    return p * total / P;
}

// Largest work-group p with start(p) <= x (x in [0, total)).
__device__ __forceinline__ long long stream_owner(long long x, long long total, long long P) {
    long long p = ((x + 1) * P - 1) / total;
    return p < P - 1 ? p : P - 1;
}

// Prefix sums of the position-range lengths (hi - lo of unit_range: the
// attended length, less what a sliding window skips) into cum[0..B]
// (cum[0] = 0), B <=
// kStreamMaxB.  Wavefront 0 does it: lane l owns sequences [16 l, 16 l + 16),
// issues all its loads at once, and a shuffle scan across the 64 lanes gives
// each lane its starting offset.  Called by the whole work-group; ends with
// a barrier.
constexpr int kScanPerLane = kStreamMaxB / 64;

__device__ inline void stream_prefix(const DecodeArgs& a, long long* cum) {
    const int tid = threadIdx.x;
    if (tid < 64) {
        const int b0 = tid * kScanPerLane;
        int len[kScanPerLane];
        // Unconditional loads (index clamped to B - 1, B >= 1) so that all of
        // them are in flight together; entries past B are zeroed afterwards.
#pragma unroll
        for (int k = 0; k < kScanPerLane; ++k) len[k] = a.seq_lens[min(b0 + k, a.B - 1)];
#pragma unroll
        for (int k = 0; k < kScanPerLane; ++k)
            if (b0 + k < a.B) {
                const PosRange r = unit_range(a, len[k]);
                len[k] = r.hi - r.lo;
            } else {
                len[k] = 0;
            }
        long long sum = 0;
#pragma unroll
        for (int k = 0; k < kScanPerLane; ++k) sum += len[k];
        long long incl = sum;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const long long y = __shfl_up(incl, off, 64);
            if (tid >= off) incl += y;
        }
        long long run = incl - sum;
#pragma unroll
        for (int k = 0; k < kScanPerLane; ++k) {
            const int b = b0 + k;
            run += len[k];
            if (b < a.B) cum[b + 1] = run;
        }
        if (tid == 0) cum[0] = 0;
    }
    __syncthreads();
}

// First sequence b with g*cum[b] <= x < g*cum[b+1] (binary search; skips
// sequences of length 0, whose range is empty).
__device__ __forceinline__ int stream_find_seq(const long long* cum, int B, int g, long long x) {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((long long)g * cum[mid] <= x) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// The work-groups holding partial records of unit (b, j): pa..pb, record slot
// 1 of pa when pa's range starts before the unit (the unit is then pa's last
// segment), slot 0 otherwise; work-groups with an empty range hold none.
struct UnitSpan {
    long long pa, pb, total, P;
    bool pa_last;
    __device__ bool empty(long long q) const {
        return stream_start(q, total, P) >= stream_start(q + 1, total, P);
    }
    __device__ long long record(long long q, int m, int r) const {
        return (q * 2 + ((q == pa && pa_last) ? 1 : 0)) * m + r;
    }
};

__device__ inline UnitSpan unit_span(const DecodeArgs& a, const long long* cum, int b, int j) {
    UnitSpan sp;
    const long long L = cum[b + 1] - cum[b];
    const long long U = (long long)a.g * cum[b] + (long long)j * L;
    sp.total = (long long)a.g * cum[a.B];
    sp.P = a.num_wgs;
    sp.pa = stream_owner(U, sp.total, sp.P);
    sp.pb = stream_owner(U + L - 1, sp.total, sp.P);
    sp.pa_last = stream_start(sp.pa, sp.total, sp.P) < U;
    return sp;
}

// Walk the segments of work-group p.  `seg(b, j, s, e, complete, slot)` is
// called once per segment, uniformly by the whole work-group.
template <class SegFn>
__device__ inline void stream_walk(const DecodeArgs& a, const long long* cum, SegFn&& seg) {
    const long long P = a.num_wgs;
    const long long total = (long long)a.g * cum[a.B];
    if (total == 0) return;
    const long long p = blockIdx.x;
    const long long start = stream_start(p, total, P);
    const long long end = stream_start(p + 1, total, P);
    if (start >= end) return;
    int b = stream_find_seq(cum, a.B, a.g, start);
    long long L = cum[b + 1] - cum[b];
    int j = (int)((start - (long long)a.g * cum[b]) / L);
    long long x = start;
    int slot = 0;
    while (x < end) {
        const long long U = (long long)a.g * cum[b] + (long long)j * L;
        const long long s = x - U;
        const long long e = (end - U) < L ? (end - U) : L;
        seg(b, j, (int)s, (int)e, s == 0 && e == L, slot);
        slot = 1;
        x = U + e;
        if (x >= end) break;
        if (++j == a.g) {
            j = 0;
            do {
                ++b;
            } while (b < a.B && cum[b + 1] == cum[b]);
            if (b >= a.B) break;
            L = cum[b + 1] - cum[b];
        }
    }
}

}  // namespace kvc
