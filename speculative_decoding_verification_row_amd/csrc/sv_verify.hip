// sv_verify.hip -- batched speculative-decoding verification for MI355X
// (gfx950, CDNA4, wave64).
//
// What is computed: the verification step of the spec-verify kernel card
// (section "Method", greedy and speculative-sampling bullets; unnormalised
// masses from its "Correctness" section).  Conventions where the card is
// silent are stated in include/sv_verify.h.
//
// Work decomposition (the vocabulary axis is the long one):
//   * every row of V values is cut into NC chunks: 4096 values in sampled
//     mode, 8192 in greedy mode.  A block has 256 threads (4 waves); each
//     thread issues coalesced 16-byte loads, all of a chunk's loads in flight
//     together, non-temporal except in the last blocks of the sampled grid
//     (a finishing block may read their chunks again soon after).
//   * greedy: one block per (row, chunk), B * (K+1) * NC blocks.  Each
//     publishes its chunk's (max, lowest-index argmax); the block of row K in
//     a column that rotates with b combines the rows of sequence b in chunk
//     order, takes the decisions, and writes n and the argmax of row n.
//   * sampled: one walk block per (sequence b, chunk column c) streams target
//     and draft rows 0..K-1 of its column, the next row loading while the
//     current one is reduced, and publishes per row its chunk's fp64 masses
//     of p and q.  The acceptance test of row i needs the row masses P_i and
//     Q_i, so the partials of all NC sibling walks, which stream the same
//     rows at the same time: a walk decides row i one step later, polling
//     its partials just before it issues row i+2's loads (loads return in
//     order, so they arrive first), and keeps row i parked in LDS meanwhile.
//     At the first rejected row n every walk publishes its chunk's residual
//     mass sum max(0, p*Q - q*P) from the parked row, then only streams.  The
//     walk of a column that rotates with b draws from the residual of row n
//     (the chunk is located from the published residual masses, then
//     searched) and publishes the sequence's outcome.  The bonus row K is
//     read by short blocks at the end of the grid (two chunks each), which
//     keep the machine busy while the last walks end; the one of the
//     rotating column finishes the sequence, drawing the bonus token from
//     p_K after full acceptance.
//   * every result depends on V alone (fixed chunking and combine order),
//     never on B, K, the launch shape or timing.
//
// Cross-block data and progress.  There are no counters and no
// read-modify-write atomics in global memory.  Every published 8-byte word
// carries the call's epoch (1..255, chosen by the host per workspace) in its
// low byte, which readers strip: the low 8 mantissa bits of an fp64 partial
// (a relative change below 2^-44, the same for every reader), the byte below
// the argmax of a (max, argmax) word, the byte below the outcome code of a
// sequence's outcome word.  The position is the same for every kind of word,
// so a word an earlier call left at an address this call reads, whatever
// its kind, shows that call's epoch.  A reader polls until each word it
// needs carries the current epoch.  If a word has not arrived within a time bound (its
// producer has not been scheduled), the reader computes that partial itself
// with the producer's arithmetic in the producer's order, so the value is
// bit-identical.  No wait is unbounded, and correctness never depends on the
// order in which workgroups are dispatched.

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <unordered_map>

#include "sv_verify.h"

#pragma clang fp contract(off)

// The workspace of sv_verify_sample_batched_noalloc, one copy per device.
// In host code this name is only a handle for hipGetSymbolAddress; the
// device address it resolves to is what the kernels receive.
static __device__ __align__(256) unsigned char scratch[SV_SCRATCH_BYTES];

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kVecS = 4;                        // float4 per thread per operand (sampled)
constexpr int kVecG = 8;                        // float4 per thread (greedy)
constexpr int kChunkS = kThreads * kVecS * 4;   // 4096 values
constexpr int kChunkG = kThreads * kVecG * 4;   // 8192 values
constexpr int kMaxNC = 128;                     // two chunks per lane of a wave
constexpr int kGroup = kWaves;                  // rows the finisher combines at a time
static_assert(SV_MAX_V == kMaxNC * kChunkS, "SV_MAX_V must match the chunk geometry");
constexpr unsigned kEpochs = 255;               // tags 1..255; 0 marks a cleared word
constexpr double kPollMicroseconds = 200.0;     // bound of a wait before recomputing
constexpr int kBonusChunks = 2;                 // bonus-row chunks per block (sampled)
constexpr unsigned kTailBlocks = 2048;          // the last two waves of 256 CUs x 4 resident blocks
constexpr unsigned kGreedyLdsPerBlock = 36864;   // 4 greedy blocks per CU (160 KB of LDS)
constexpr unsigned kGreedyUncappedBlocks = 2048; // 256 CUs x 8 greedy blocks: smaller grids stay uncapped
constexpr uint64_t kRowsBlocksPerRow = 512;     // one block per sampled draft row up to 512 * max(4, K) blocks
constexpr uint64_t kRowsBlocksPerRowL = 256;    // the same for logits: 256 * max(4, K)

struct Header {              // 256 bytes
    unsigned error;          // fault word (reserved: nothing in this version sets it)
    unsigned slow_path;      // 1 once a reader has recomputed a partial
    unsigned pad[62];
};

struct Part {                // 32 bytes, one per (row, chunk); tagged words
    unsigned long long sp, sq, smin;   // fp64 chunk sums of p, q, min(p, q)
    unsigned long long am;             // max value (high 32 bits), argmax (bits 8..31)
};

struct Layout {
    size_t hdr, parts, wpart, sstate, total;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline int chunk_of(bool sampled) { return sampled ? kChunkS : kChunkG; }

inline Layout make_layout(int64_t B, int64_t K, int64_t NC, bool sampled)
{
    Layout L{};
    size_t o = 0;
    L.hdr = o;   o = align_up(o + sizeof(Header), 256);
    L.parts = o; o = align_up(o + (size_t)(B * (K + 1) * NC) * sizeof(Part), 256);
    L.wpart = o; o = align_up(o + (sampled ? (size_t)(B * K * NC) * 8 : 0), 256);
    L.sstate = o; o = align_up(o + (sampled ? (size_t)B * 8 : 0), 256);
    L.total = o;
    return L;
}

struct Args {
    const float* tp;
    const float* dp;
    const int32_t* dt;
    const float* u;
    int32_t* n_out;
    int32_t* next_out;
    sv_row_stats* stats;
    Header* hdr;
    Part* parts;
    unsigned long long* wpart;       // residual chunk masses (sampled)
    unsigned long long* sstate;      // per-sequence outcome of the walks (sampled)
    unsigned nwalk;                  // sampled: blocks that walk the draft rows
    int B, K, V, NC;
    unsigned epoch;                  // this call's tag, 1..255
    int force_recompute;             // test hook: readers recompute every partial
    unsigned long long poll_ticks;   // wait bound in wall-clock ticks
    float ktau;                      // logits: log2(e) / temperature
    double ktau64;                   // the same in fp64 (acceptance weights)
    int early;                       // sampled: read no row a decided sequence no longer needs
    int force_lost;                  // test hook: every in-walk decision gives up (readers still trust partials)
};

// ------------------------------------------- cross-block communication --

// Published words are written and read with agent-scope atomic accesses,
// which gfx950 performs at the device-coherent level (no per-XCD L2 copy is
// involved, so no cache write-back or invalidate is needed).  Each word
// validates itself through its tag, so no ordering between words is needed.

__device__ __forceinline__ void put_u64(void* p, unsigned long long v)
{
    __hip_atomic_store(static_cast<unsigned long long*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long get_u64(const void* p)
{
    return __hip_atomic_load(static_cast<const unsigned long long*>(p), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_u32(void* p, unsigned v)
{
    __hip_atomic_store(static_cast<unsigned*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned long long tag_f64(double v, unsigned ep)
{
    return ((unsigned long long)__double_as_longlong(v) & ~0xFFull) | ep;
}
__device__ __forceinline__ bool f64_ok(unsigned long long w, unsigned ep) { return (w & 0xFFull) == ep; }
__device__ __forceinline__ double f64_of(unsigned long long w)
{
    return __longlong_as_double((long long)(w & ~0xFFull));
}
// the value every reader obtains for a published fp64 partial
__device__ __forceinline__ double strip8(double v) { return f64_of((unsigned long long)__double_as_longlong(v)); }

// A (value, argmax) word: the value's bits in the high 32 bits, the argmax
// (24 bits; positions are below 2^19) in bits 8..31, and the tag in the low
// byte like every other published word.  One tag position for every kind of
// word matters: workspace addresses serve different layouts from call to
// call, so a reader may find, where it expects its word, a word another
// call left there of another kind; that word's low byte is then that call's
// tag, never this call's.
__device__ __forceinline__ unsigned long long tag_am(float v, int arg, unsigned ep)
{
    return ((unsigned long long)__float_as_uint(v) << 32) | ((unsigned long long)((unsigned)arg & 0xFFFFFFu) << 8) |
           ep;
}
__device__ __forceinline__ bool am_ok(unsigned long long w, unsigned ep) { return (w & 0xFFull) == ep; }
__device__ __forceinline__ float am_val(unsigned long long w) { return __uint_as_float((unsigned)(w >> 32)); }
__device__ __forceinline__ int am_arg(unsigned long long w) { return (int)((w >> 8) & 0xFFFFFFu); }

// An empty asm that takes a value and gives it back.  Applied to polled
// values once the step's row loads are issued, it keeps the compiler from
// moving what is computed from them (the fp64 conversions of the acceptance
// test) up to the polls themselves: waiting there, one poll after another,
// would hold back the wave's row loads by as many round trips to memory.
// Applied to the thread index, it keeps what is computed from it where it
// is written, instead of hoisted out of a loop and held (or spilled) there.
template <class T>
__device__ __forceinline__ void settle(T& v)
{
    asm volatile("" : "+v"(v));
}

// Block-uniform bounded wait: true once the bound has passed (thread 0's
// clock decides, so every thread leaves the wait loop together).
__device__ __forceinline__ bool wait_expired(const Args& a, unsigned long long t0)
{
    return __syncthreads_or(threadIdx.x == 0 && (a.force_recompute || wall_clock64() - t0 > a.poll_ticks));
}

// ---------------------------------------------------------- chunk I/O --

// Rows are read through buffer resources: the row's base address lives in
// scalar registers and each thread keeps one 32-bit byte offset, and the
// resource's range check returns 0 for every value at index V or beyond
// without touching memory.  Those zeros cannot change a sum, and they cannot
// become the argmax (values are non-negative and the lowest index wins a
// tie), so no masking is needed anywhere.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kRsrcWord3 = 0x00020000;   // gfx9 raw buffer: 32-bit data format
constexpr int kNonTemporal = 2;          // cache policy bit: streamed, not kept

struct Row {
    __amdgpu_buffer_rsrc_t r;
};

__device__ __forceinline__ Row row_of(const float* base, int V)
{
    return Row{__builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, V * 4, kRsrcWord3)};
}

// Thread t holds float4 number (c * 256 * NV + k * 256 + t) of the row,
// k < NV: consecutive threads read consecutive 16-byte words (coalesced).
template <int NV>
__device__ __forceinline__ int f4_index(int c, int k) { return c * (kThreads * NV) + k * kThreads + (int)threadIdx.x; }

__device__ __forceinline__ float4 as_float4(u32x4 v)
{
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}

// Streaming loads of float4 numbers k in [0, NV) of chunk c; all of a
// thread's loads are issued back to back and stay in flight together.  The
// scalar form (rows not 16-byte aligned, or V not a multiple of 4) reads
// the same values one float at a time.  AUX is the cache policy.
template <bool VEC, int NV, int AUX = kNonTemporal>
__device__ __forceinline__ void load_chunk(Row row, int c, float4 (&v)[NV])
{
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int off = f4_index<NV>(c, k) * 16;
        if constexpr (VEC) {
            v[k] = as_float4(__builtin_amdgcn_raw_buffer_load_b128(row.r, off, 0, AUX));
        } else {
            float e[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                e[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(row.r, off + 4 * j, 0, AUX));
            v[k] = make_float4(e[0], e[1], e[2], e[3]);
        }
    }
}

// The same loads, kept in the caches when `keep`: for the last blocks of the
// grid, whose chunks a finishing block may read again soon after.
template <bool VEC, int NV>
__device__ __forceinline__ void load_chunk_keep(Row row, int c, float4 (&v)[NV], bool keep)
{
    if (keep)
        load_chunk<VEC, NV, 0>(row, c, v);
    else
        load_chunk<VEC, NV>(row, c, v);
}

// Cached load of float4 number k (runtime) of chunk c.
template <bool VEC, int NV>
__device__ __forceinline__ float4 load_one(Row row, int c, int k)
{
    const int off = f4_index<NV>(c, k) * 16;
    if constexpr (VEC) {
        return as_float4(__builtin_amdgcn_raw_buffer_load_b128(row.r, off, 0, 0));
    } else {
        float e[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) e[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(row.r, off + 4 * j, 0, 0));
        return make_float4(e[0], e[1], e[2], e[3]);
    }
}

__device__ __forceinline__ float comp(float4 v, int e)
{
    return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
}

// Residual mass of one value: max(0, p*Q - q*P), fp64, no contraction.
__device__ __forceinline__ double resid(float p, float q, double P, double Q)
{
    const double d = (double)p * Q - (double)q * P;
    return d > 0.0 ? d : 0.0;
}

// ------------------------------------------------------- reductions --

// Which statistics a pass accumulates and publishes for a chunk.  The masses
// P and Q decide acceptance, the argmax decides greedy verification, and the
// remaining fields exist only for the optional per-row statistics output, so
// a call without statistics leaves them out of the streamed pass.
enum : int { kSP = 1, kSQ = 2, kSMIN = 4, kAM = 8 };

struct Acc {
    double sp, sq, smin;
    float maxv;
    int arg;
};

// (value, index) order: larger value first, then lower index (lowest-index
// argmax).  A total order, so any merge tree gives the same result.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float ov, int oi)
{
    if (ov > v || (ov == v && oi < i)) {
        v = ov;
        i = oi;
    }
}

// Adds float4 number k of the thread's chunk share.  This is the single
// definition of the per-thread order: the streamed path and the recompute
// path both call it, and each field's sum is independent of which other
// fields are accumulated.  While a thread accumulates, arg holds the
// position 4k + e of its maximum among its own values (positions increase
// with the index, so the first maximum is the lowest index); thread_arg()
// turns it into the row index.
template <int M>
__device__ __forceinline__ void acc_f4(Acc& a, float4 p4, float4 q4, int k)
{
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float p = comp(p4, e);
        if constexpr ((M & kAM) != 0) {
            if (p > a.maxv) {
                a.maxv = p;
                a.arg = 4 * k + e;
            }
        }
        if constexpr ((M & kSP) != 0) a.sp += (double)p;
        if constexpr ((M & (kSQ | kSMIN)) != 0) {
            const double qd = (double)comp(q4, e);
            if constexpr ((M & kSQ) != 0) a.sq += qd;
            if constexpr ((M & kSMIN) != 0) a.smin += __builtin_fmin((double)p, qd);
        }
    }
}

// Row index of the thread-local position 4k + e in chunk c.
template <int NV>
__device__ __forceinline__ void thread_arg(Acc& a, int c)
{
    a.arg = f4_index<NV>(c, a.arg >> 2) * 4 + (a.arg & 3);
}

template <int M, int NV>
__device__ __forceinline__ Acc thread_stats(const float4 (&pv)[NV], const float4 (&qv)[NV], int c)
{
    Acc a{0.0, 0.0, 0.0, -INFINITY, 0};
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        acc_f4<M>(a, pv[k], qv[k], k);
        __builtin_amdgcn_sched_barrier(0);   // keep fp64 temporaries to one float4 at a time
    }
    thread_arg<NV>(a, c);
    return a;
}

// The same per-thread sums, re-reading the chunk one float4 at a time.
template <bool VEC, int M, int NV>
__device__ __forceinline__ Acc thread_stats_reload(Row prow, Row qrow, int c)
{
    constexpr bool kQ = (M & (kSQ | kSMIN)) != 0;
    Acc a{0.0, 0.0, 0.0, -INFINITY, 0};
    for (int k = 0; k < NV; ++k) {
        const float4 p4 = load_one<VEC, NV>(prow, c, k);
        const float4 q4 = kQ ? load_one<VEC, NV>(qrow, c, k) : p4;
        acc_f4<M>(a, p4, q4, k);
    }
    thread_arg<NV>(a, c);
    return a;
}

__device__ __forceinline__ double resid_f4(float4 p4, float4 q4, double P, double Q)
{
    double w = 0.0;
#pragma unroll
    for (int e = 0; e < 4; ++e) w += resid(comp(p4, e), comp(q4, e), P, Q);
    return w;
}

template <bool VEC, int NV>
__device__ __forceinline__ double thread_resid_reload(Row prow, Row qrow, int c, double P, double Q)
{
    double w = 0.0;
    for (int k = 0; k < NV; ++k) w += resid_f4(load_one<VEC, NV>(prow, c, k), load_one<VEC, NV>(qrow, c, k), P, Q);
    return w;
}

// Wave-level exchanges through DPP (data-parallel primitives: a lane reads
// another lane of its 16-lane row inside a VALU move, no LDS round trip).
// Controls: swap within pairs, swap pairs within quads, mirror within
// halves of a row, mirror within a row.  After the four steps every lane of
// a row holds the row's result (each step combines a lane with its partner,
// and the two partners compute the same commutative sum or merge).
constexpr int kDppPairs = 0xB1, kDppQuads = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

// Every control used with it gives every lane a source lane (the four above
// permute a row; quad broadcasts such as 0x55, lane 1 of each quad to the
// whole quad, are used too), so the move needs no prior value in its
// destination: a plain DPP move, not an update of a zeroed register (one
// VALU move fewer per step).
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v)
{
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v)
{
    const long long bits = __double_as_longlong(v);
    const int lo = dpp_i32<CTRL>((int)bits), hi = dpp_i32<CTRL>((int)(bits >> 32));
    return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// Exchanges across the wave's four 16-lane rows by gfx950's lane swaps
// (v_permlane16_swap, v_permlane32_swap), in vector registers: rows_01_23(v)
// gives the lanes of rows 0 and 1 the pair (row 0's, row 1's value) and the
// lanes of rows 2 and 3 (row 2's, row 3's); halves(v) gives every lane
// (lanes 0..31's, lanes 32..63's value).  Applied to values that are equal
// across each row, they combine four row results r0..r3 as (r0 . r1) .
// (r2 . r3) in every lane: the order the scalar reads of lanes 0, 16, 32, 48
// gave, without those reads (logits 229.1 -> 227.9 us, statistics 237.4 ->
// 235.4 us at B=256 K=5 V=128256 together with the plain DPP moves above).
__device__ __forceinline__ void rows_01_23(unsigned v, unsigned& a, unsigned& b)
{
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    a = r[0];
    b = r[1];
}
__device__ __forceinline__ void halves(unsigned v, unsigned& a, unsigned& b)
{
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    a = r[0];
    b = r[1];
}
template <bool HALVES>
__device__ __forceinline__ void swap_f64(double v, double& a, double& b)
{
    const unsigned long long bits = (unsigned long long)__double_as_longlong(v);
    unsigned al, ah, bl, bh;
    if constexpr (HALVES) {
        halves((unsigned)bits, al, bl);
        halves((unsigned)(bits >> 32), ah, bh);
    } else {
        rows_01_23((unsigned)bits, al, bl);
        rows_01_23((unsigned)(bits >> 32), ah, bh);
    }
    a = __longlong_as_double((long long)(((unsigned long long)ah << 32) | al));
    b = __longlong_as_double((long long)(((unsigned long long)bh << 32) | bl));
}

// Sum over the wave (all 64 lanes active), the same value in every lane:
// row sums by DPP, then the four row sums as (r0 + r1) + (r2 + r3).
__device__ __forceinline__ double wave_sum(double v)
{
    v += dpp_f64<kDppPairs>(v);
    v += dpp_f64<kDppQuads>(v);
    v += dpp_f64<kDppHalfMirror>(v);
    v += dpp_f64<kDppMirror>(v);
    double a, b;
    swap_f64<false>(v, a, b);
    swap_f64<true>(a + b, a, b);
    return a + b;
}

template <int CTRL>
__device__ __forceinline__ void argmax_step(float& v, int& i)
{
    const float ov = __int_as_float(dpp_i32<CTRL>(__float_as_int(v)));
    const int oi = dpp_i32<CTRL>(i);
    argmax_merge(v, i, ov, oi);
}

// (value, index) maximum over the wave (all 64 lanes active), the same in
// every lane.  The rows' results merge as (r0 . r1) . (r2 . r3) by the lane
// swaps; the merge (larger value, then lower index) is associative on finite
// values, so this is the pair the row-order scan of lanes 0, 16, 32, 48 gave
// (greedy 115.5 -> 115.0 us at B=256 K=5 V=128256).
__device__ __forceinline__ void wave_argmax(float& v, int& i)
{
    argmax_step<kDppPairs>(v, i);
    argmax_step<kDppQuads>(v, i);
    argmax_step<kDppHalfMirror>(v, i);
    argmax_step<kDppMirror>(v, i);
    unsigned av, bv, ai, bi;
    rows_01_23(__float_as_uint(v), av, bv);
    rows_01_23((unsigned)i, ai, bi);
    float mv = __uint_as_float(av);
    int mi = (int)ai;
    argmax_merge(mv, mi, __uint_as_float(bv), (int)bi);
    halves(__float_as_uint(mv), av, bv);
    halves((unsigned)mi, ai, bi);
    v = __uint_as_float(av);
    i = (int)ai;
    argmax_merge(v, i, __uint_as_float(bv), (int)bi);
}

__device__ __forceinline__ double wave_inclusive_scan(double v)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const double y = __shfl_up(v, d);
        if (lane >= d) v += y;
    }
    return v;
}

// Block reduction of the fields in M; the result is valid in thread 0.
// With TRAIL it ends with a barrier, so the block may call it again at once.
// Without, the caller alternates `slot` between consecutive calls: a slot is
// written again only two calls later, after every wave, thread 0 included
// (which has read it by then), has passed the barrier of the call between.
template <int M, bool TRAIL = true>
__device__ __forceinline__ Acc block_reduce(Acc a, int slot = 0)
{
    __shared__ double s_sp[2][kWaves], s_sq[2][kWaves], s_sm[2][kWaves];
    __shared__ float s_v[2][kWaves];
    __shared__ int s_i[2][kWaves];
    if constexpr ((M & kSP) != 0) a.sp = wave_sum(a.sp);
    if constexpr ((M & kSQ) != 0) a.sq = wave_sum(a.sq);
    if constexpr ((M & kSMIN) != 0) a.smin = wave_sum(a.smin);
    if constexpr ((M & kAM) != 0) wave_argmax(a.maxv, a.arg);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) {
        s_sp[slot][w] = a.sp;
        s_sq[slot][w] = a.sq;
        s_sm[slot][w] = a.smin;
        s_v[slot][w] = a.maxv;
        s_i[slot][w] = a.arg;
    }
    __syncthreads();
    Acc r = a;
    if (threadIdx.x == 0) {
        r = Acc{s_sp[slot][0], s_sq[slot][0], s_sm[slot][0], s_v[slot][0], s_i[slot][0]};
        for (int j = 1; j < kWaves; ++j) {
            r.sp += s_sp[slot][j];
            r.sq += s_sq[slot][j];
            r.smin += s_sm[slot][j];
            argmax_merge(r.maxv, r.arg, s_v[slot][j], s_i[slot][j]);
        }
    }
    if (TRAIL) __syncthreads();
    return r;
}

// Block sum; the result is valid in thread 0.  Ends with a barrier.
__device__ __forceinline__ double block_sum(double v)
{
    __shared__ double s[kWaves];
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = v;
    __syncthreads();
    double r = v;
    if (threadIdx.x == 0) {
        r = s[0];
        for (int j = 1; j < kWaves; ++j) r += s[j];
    }
    __syncthreads();
    return r;
}

// Wave-cooperative sum of chunk values s[0..NC) in a fixed order: lane l
// adds chunks l and l + 64, then a butterfly.  Every reader of a row uses
// this one order, so all of them obtain the same row masses.
__device__ __forceinline__ double sum_chunks(const double* s, int NC)
{
    const int lane = threadIdx.x & 63;
    const double v = (lane < NC ? s[lane] : 0.0) + (lane + 64 < NC ? s[lane + 64] : 0.0);
    return wave_sum(v);
}

// The acceptance test of a draft token (fp64, scale-free): accept iff
// u * q(t) * P < p(t) * Q.  Every place that decides uses this expression.
__device__ __forceinline__ bool accepted(float u, double pt, double qt, double P, double Q)
{
    return (double)u * (double)qt * P < (double)pt * Q;
}

// Publish the fields in M of a chunk's reduced statistics (thread 0).
template <int M>
__device__ __forceinline__ void publish_part(const Args& a, int64_t row, int c, const Acc& s)
{
    if (threadIdx.x == 0) {
        Part* dst = &a.parts[row * a.NC + c];
        if constexpr ((M & kSP) != 0) put_u64(&dst->sp, tag_f64(s.sp, a.epoch));
        if constexpr ((M & kSQ) != 0) put_u64(&dst->sq, tag_f64(s.sq, a.epoch));
        if constexpr ((M & kSMIN) != 0) put_u64(&dst->smin, tag_f64(s.smin, a.epoch));
        if constexpr ((M & kAM) != 0) put_u64(&dst->am, tag_am(s.maxv, s.arg, a.epoch));
    }
}

// ------------------------------------------------------ gathering --

// The gathered partials of up to kGroup rows of one sequence (LDS), for at
// most NCMAX chunks per row.
template <int NCMAX>
struct Gathered {
    static constexpr int kCap = NCMAX;
    double sp[kGroup][NCMAX];
    double sq[kGroup][NCMAX];
    double smin[kGroup][NCMAX];
    unsigned long long am[kGroup][NCMAX];
};

// LDS of a block: while it walks its chunk column, the chunk of the row
// whose decision is pending (target float4s, then draft float4s; each thread
// touches only its own column, so no barrier guards it); when it finishes a
// sequence, the gathered partials.
// The partials of several rows of one sequence, entry r * NC + c for row r
// of the tile and chunk c.
struct FlatGathered {
    static constexpr int kCap = kGroup * kMaxNC;
    double sp[kCap], sq[kCap], smin[kCap];
    unsigned long long am[kCap];
};

union SampleLds {
    f32x4 parked[2 * kVecS][kThreads];
    Gathered<kMaxNC> g;
    FlatGathered f;
};
__shared__ SampleLds lds;
// The greedy kernel's rows have at most SV_MAX_V / kChunkG chunks.
__shared__ Gathered<SV_MAX_V / kChunkG> lds_greedy;

template <int M, class G>
__device__ __forceinline__ bool part_ok(G& g, const Part* pp, unsigned ep, int r, int c, bool store)
{
    const unsigned long long wsp = (M & kSP) ? get_u64(&pp->sp) : 0ull;
    const unsigned long long wsq = (M & kSQ) ? get_u64(&pp->sq) : 0ull;
    const unsigned long long wsm = (M & kSMIN) ? get_u64(&pp->smin) : 0ull;
    const unsigned long long wam = (M & kAM) ? get_u64(&pp->am) : 0ull;
    const bool ok = (!(M & kSP) || f64_ok(wsp, ep)) && (!(M & kSQ) || f64_ok(wsq, ep)) &&
                    (!(M & kSMIN) || f64_ok(wsm, ep)) && (!(M & kAM) || am_ok(wam, ep));
    if (ok && store) {
        g.sp[r][c] = f64_of(wsp);
        g.sq[r][c] = f64_of(wsq);
        g.smin[r][c] = f64_of(wsm);
        g.am[r][c] = wam;
    }
    return ok;
}

template <bool VEC, int M, int NV, class G>
__device__ void recompute_part(G& g, const Args& a, Row prow, Row qrow, int r, int c)
{
    const Acc s = block_reduce<M>(thread_stats_reload<VEC, M, NV>(prow, qrow, c));
    if (threadIdx.x == 0) {
        g.sp[r][c] = strip8(s.sp);
        g.sq[r][c] = strip8(s.sq);
        g.smin[r][c] = strip8(s.smin);
        g.am[r][c] = tag_am(s.maxv, s.arg, a.epoch);
        put_u32(&a.hdr->slow_path, 1u);
    }
}

// Block-cooperative: read the partials of rows row0 .. row0 + nrows - 1 of
// sequence b (rows numbered within the sequence) into g: fields MROW of
// rows below K and MLAST of row K.  Partials that do not carry this call's
// tag within the wait bound are recomputed from the inputs.
template <bool VEC, int NV, int MROW, int MLAST, class G>
__device__ void gather_rows(G& g, const Args& a, int b, int row0, int nrows)
{
    __shared__ unsigned long long s_miss[kGroup][2];
    const int NC = a.NC, K = a.K, V = a.V;
    const unsigned ep = a.epoch;
    const int n_ent = nrows * NC;
    constexpr int kPer = (kGroup * G::kCap + kThreads - 1) / kThreads;   // entries per thread
    bool need[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) need[j] = (int)threadIdx.x + j * kThreads < n_ent;
    const unsigned long long t0 = wall_clock64();
    for (;;) {
        bool any = false;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            if (!need[j]) continue;
            const int e = (int)threadIdx.x + j * kThreads, r = e / NC, c = e - r * NC;
            const int i = row0 + r;
            const Part* pp = &a.parts[((int64_t)b * (K + 1) + i) * NC + c];
            const bool ok = i < K ? part_ok<MROW>(g, pp, ep, r, c, !a.force_recompute)
                                  : part_ok<MLAST>(g, pp, ep, r, c, !a.force_recompute);
            if (ok && !a.force_recompute)
                need[j] = false;
            else
                any = true;
        }
        if (!__syncthreads_or(any)) return;   // everything arrived (the usual case)
        if (wait_expired(a, t0)) break;
        __builtin_amdgcn_s_sleep(2);
    }
    // what is still missing (rare): recompute it, one chunk at a time
    if (threadIdx.x < kGroup * 2) s_miss[threadIdx.x >> 1][threadIdx.x & 1] = 0ull;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        if (!need[j]) continue;
        const int e = (int)threadIdx.x + j * kThreads, r = e / NC, c = e - r * NC;
        atomicOr(&s_miss[r][c >> 6], 1ull << (c & 63));   // LDS
    }
    __syncthreads();
    for (int r = 0; r < nrows; ++r) {
        const int i = row0 + r;
        const int64_t row = (int64_t)b * (K + 1) + i;
        const Row prow = row_of(a.tp + row * V, V);
        const bool has_q = i < K && (MROW & (kSQ | kSMIN)) != 0;
        const Row qrow = has_q ? row_of(a.dp + ((int64_t)b * K + i) * V, V) : prow;
        for (int h = 0; h < 2; ++h) {
            unsigned long long mk = s_miss[r][h];
            while (mk) {
                const int c = h * 64 + __ffsll((unsigned long long)mk) - 1;
                mk &= mk - 1;
                if (i < K)
                    recompute_part<VEC, MROW, NV>(g, a, prow, qrow, r, c);
                else
                    recompute_part<VEC, MLAST, NV>(g, a, prow, qrow, r, c);
            }
        }
    }
    __syncthreads();
}

// Wave-cooperative combine of gathered row r (values valid in every lane).
struct RowView {
    double P, Q, Smin;
    float maxv;
    int arg;
};

template <int M, class G>
__device__ __forceinline__ RowView combine_row(const G& g, int r, int NC)
{
    const int lane = threadIdx.x & 63;
    RowView v{0.0, 0.0, 0.0, -INFINITY, INT_MAX};
    if constexpr ((M & kSP) != 0) v.P = sum_chunks(g.sp[r], NC);
    if constexpr ((M & kSQ) != 0) v.Q = sum_chunks(g.sq[r], NC);
    if constexpr ((M & kSMIN) != 0) v.Smin = sum_chunks(g.smin[r], NC);
    if constexpr ((M & kAM) != 0) {
        float mv = -INFINITY;
        int ai = INT_MAX;
        for (int h = 0; h < 2; ++h) {
            const int c = lane + 64 * h;
            if (c < NC) argmax_merge(mv, ai, am_val(g.am[r][c]), am_arg(g.am[r][c]));
        }
        wave_argmax(mv, ai);
        v.maxv = mv;
        v.arg = ai;
    }
    return v;
}

// ---------------------------------------------------- inverse CDF --

// Wave-cooperative: given chunk masses m[0..NC) (chunks 2l and 2l+1 in lane
// l), the chunk c with prefix(c-1) <= T < prefix(c) for T = u * total, and
// its base prefix(c-1).  Prefixes are an inclusive scan in chunk order and
// the total is its last entry, so T < total always has an owner when
// total > 0.  Returns the total; *owner = -1 when total == 0.
__device__ __forceinline__ double locate_chunk(const double* m, int NC, double u, int* owner, double* base,
                                               double* T_out)
{
    const int lane = threadIdx.x & 63;
    const int c0 = 2 * lane, c1 = 2 * lane + 1;
    const double m0 = c0 < NC ? m[c0] : 0.0, m1 = c1 < NC ? m[c1] : 0.0;
    const double incl = wave_inclusive_scan(m0 + m1);
    const double total = __shfl(incl, 63);
    const double T = u * total;
    double lo = __shfl_up(incl, 1);
    if (lane == 0) lo = 0.0;
    const double mid = lo + m0;
    const bool own0 = c0 < NC && lo <= T && T < mid;
    const bool own1 = c1 < NC && !own0 && mid <= T && T < incl;
    const unsigned long long mk = __ballot(own0 || own1);
    int c = -1;
    double bs = 0.0;
    if (mk) {
        const int l = __ffsll((unsigned long long)mk) - 1;
        const int which = __shfl(own0 ? 0 : 1, l);
        const double lo_l = __shfl(lo, l), mid_l = __shfl(mid, l);
        c = 2 * l + which;
        bs = which == 0 ? lo_l : mid_l;
    }
    *owner = c;
    *base = bs;
    *T_out = T;
    return total;
}

// Search of chunk c for the smallest x with
// base + sum_{chunk start <= y <= x} w(y) > T, where w is the residual
// max(0, p*Q - q*P) (RESID) or p itself.  If rounding leaves no such x in
// the chunk, the last x with w(x) > 0 is taken.  Each thread loads its whole
// share of the chunk at once; segment (k, wave) is 256 consecutive values
// and segments are in index order: the segment masses locate the segment,
// and the wave that holds it scans its values.  All threads of the block
// must call; the token is returned in every thread.
template <bool VEC, bool RESID, int NV>
__device__ __forceinline__ int chunk_draw(Row prow, Row qrow, double P, double Q, int c, double base, double T)
{
    __shared__ double s_seg[NV][kWaves];
    __shared__ int s_ks, s_ws;
    __shared__ double s_base;
    __shared__ int s_x;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;

    auto wsum4 = [&](float4 p4, float4 q4) -> double {   // one float4, in index order
        double t = 0.0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            t += RESID ? resid(comp(p4, e), comp(q4, e), P, Q) : (double)comp(p4, e);
        return t;
    };

    float4 pv[NV], qv[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        pv[k] = load_one<VEC, NV>(prow, c, k);
        qv[k] = RESID ? load_one<VEC, NV>(qrow, c, k) : pv[k];
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const double s = wave_sum(wsum4(pv[k], qv[k]));
        if (lane == 0) s_seg[k][w] = s;
    }
    __syncthreads();
    if (threadIdx.x < 64) {
        // segment q = k * kWaves + j in lane q: the first segment whose
        // running mass passes T (or, by rounding only, the last with mass)
        constexpr int kSegs = NV * kWaves;
        const int q = threadIdx.x;
        const double s = q < kSegs ? s_seg[q / kWaves][q % kWaves] : 0.0;
        const double incl = wave_inclusive_scan(s);
        double excl = __shfl_up(incl, 1);
        if (q == 0) excl = 0.0;
        const double run = base + excl;
        const unsigned long long mh = __ballot(q < kSegs && run + s > T);
        const unsigned long long mp = __ballot(q < kSegs && s > 0.0);
        const int sel = mh ? __ffsll((unsigned long long)mh) - 1 : (mp ? 63 - __clzll(mp) : 0);
        const double bs = __shfl(run, sel);
        if (q == 0) {
            s_ks = sel / kWaves;
            s_ws = sel % kWaves;
            s_base = bs;
        }
    }
    __syncthreads();
    if (w == s_ws) {
        const int k = s_ks;
        float4 p4 = pv[0], q4 = qv[0];
#pragma unroll
        for (int kk = 1; kk < NV; ++kk)
            if (kk == k) {
                p4 = pv[kk];
                q4 = qv[kk];
            }
        const double incl = wave_inclusive_scan(wsum4(p4, q4));
        double run = __shfl_up(incl, 1);
        if (lane == 0) run = 0.0;
        run += s_base;
        int hit = -1, lastpos = -1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const double v = RESID ? resid(comp(p4, e), comp(q4, e), P, Q) : (double)comp(p4, e);
            run += v;
            if (hit < 0 && run > T) hit = e;
            if (v > 0.0) lastpos = e;
        }
        const unsigned long long mh = __ballot(hit >= 0);
        if (mh) {
            const int l = __ffsll((unsigned long long)mh) - 1;
            if (lane == l) s_x = f4_index<NV>(c, k) * 4 + hit;
        } else {
            const unsigned long long mp = __ballot(lastpos >= 0);
            if (mp) {
                const int l = 63 - __clzll(mp);
                if (lane == l) s_x = f4_index<NV>(c, k) * 4 + lastpos;
            } else if (lane == 0) {
                s_x = f4_index<NV>(c, k) * 4;   // unreachable for a segment with mass
            }
        }
    }
    __syncthreads();
    return s_x;
}

__device__ __forceinline__ void write_stats(const Args& a, int64_t row, const RowView& rv, bool pair,
                                            float pt, float qt, bool has_t)
{
    sv_row_stats s;
    s.argmax = rv.arg;
    s.max_p = rv.maxv;
    s.sum_p = rv.P;
    s.sum_q = pair ? rv.Q : 0.0;
    s.sum_min = pair ? rv.Smin : 0.0;
    s.sum_pos = pair ? rv.P - rv.Smin : 0.0;
    s.p_t = has_t ? pt : 0.0f;
    s.q_t = pair ? qt : 0.0f;
    a.stats[row] = s;
}

// -------------------------------------------------------- finishing --

// The column whose block finishes sequence b.  Workgroups are handed to the
// eight XCDs round-robin by index, so a fixed column would put every
// sequence's finishing work on one XCD; rotating it with b spreads that work
// over all of them.
__device__ __forceinline__ int finisher_column(int b, int NC) { return b % NC; }

struct Outcome {
    int n;          // accept-prefix length
    double P, Q;    // masses of row n
    int arg;        // argmax of row n
};

// Block-cooperative, run by the finishing block of sequence b after its walk:
// combine the rows of sequence b in groups of kGroup (wave w takes row
// g0 + w), take the decisions and, when `write` is set, write the row
// statistics; without it it stops after the group that holds the first
// rejection.  Uniform result.
template <bool VEC, bool SAMPLED, int NV, int MROW, int MLAST, class G>
__device__ Outcome finish_rows(G& g, const Args& a, int b, bool write)
{
    __shared__ int s_rej[kGroup], s_arg[kGroup];
    __shared__ double s_P[kGroup], s_Q[kGroup];
    const int K = a.K, V = a.V, NC = a.NC;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    Outcome o{K, 0.0, 0.0, 0};
    bool done = false;
    for (int g0 = 0; g0 <= K; g0 += kGroup) {
        const int nrows = (K + 1 - g0) < kGroup ? (K + 1 - g0) : kGroup;
        const int i = g0 + w;
        // The token of row i loads while the partials are gathered, its
        // values and the uniform while the row is combined; the values are
        // settled (waited for) only after that, together.
        int tk = -1;
        if (w < nrows && lane == 0 && i < K) tk = a.dt[(int64_t)b * K + i];
        gather_rows<VEC, NV, MROW, MLAST>(g, a, b, g0, nrows);
        if (w < nrows) {
            const int64_t row = (int64_t)b * (K + 1) + i;
            const bool pair = SAMPLED && i < K;
            const bool tin = tk >= 0 && tk < V;
            float pt = 0.0f, qt = 0.0f, u = 0.0f;
            if (lane == 0 && (SAMPLED || write)) {
                const int64_t x = tin ? tk : 0;
                pt = a.tp[row * V + x];
                if (pair) {
                    qt = a.dp[((int64_t)b * K + i) * V + x];
                    u = a.u[row];
                }
            }
            const RowView rv = i < K ? combine_row<MROW>(g, w, NC) : combine_row<MLAST>(g, w, NC);
            if (lane == 0) {
                settle(pt);
                settle(qt);
                settle(u);
                if (!tin) {
                    pt = 0.0f;
                    qt = 0.0f;
                }
                int rej = 0;
                if (SAMPLED) {
                    if (pair) rej = accepted(u, pt, qt, rv.P, rv.Q) ? 0 : 1;
                } else {
                    rej = (i < K && tk != rv.arg) ? 1 : 0;
                }
                if (write) write_stats(a, row, rv, pair, pt, qt, i < K);
                s_rej[w] = rej;
                s_P[w] = rv.P;
                s_Q[w] = rv.Q;
                s_arg[w] = rv.arg;
            }
        }
        __syncthreads();
        if (!done) {
            int pick = -1;
            for (int r = 0; r < nrows; ++r)
                if (pick < 0 && s_rej[r]) pick = r;
            if (pick < 0 && g0 + nrows == K + 1) pick = nrows - 1;   // row K: every draft accepted
            if (pick >= 0) {
                o = Outcome{g0 + pick, s_P[pick], s_Q[pick], s_arg[pick]};
                done = true;
            }
        }
        __syncthreads();
        if (done && !write) break;
    }
    return o;
}

// Block-cooperative: the partials of rows row0 .. row0 + nrows - 1 of sequence
// b into f (fields MROW of rows below K, MLAST of row K), nrows * NC <=
// FlatGathered::kCap.  Partials that do not carry this call's tag within the
// wait bound are recomputed from the inputs (as gather_rows does).
template <bool VEC, int MROW, int MLAST>
__device__ void gather_flat(FlatGathered& f, const Args& a, int b, int row0, int nrows)
{
    constexpr int kPer = FlatGathered::kCap / kThreads;
    const int NC = a.NC, K = a.K, V = a.V;
    const unsigned ep = a.epoch;
    const int n_ent = nrows * NC;
    bool need[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) need[j] = (int)threadIdx.x + j * kThreads < n_ent;
    const unsigned long long t0 = wall_clock64();
    for (;;) {
        bool any = false;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            if (!need[j]) continue;
            const int e = (int)threadIdx.x + j * kThreads, r = e / NC, c = e - r * NC;
            const int i = row0 + r;
            const Part* pp = &a.parts[((int64_t)b * (K + 1) + i) * NC + c];
            const int M = i < K ? MROW : MLAST;
            const unsigned long long wsp = get_u64(&pp->sp);
            const unsigned long long wsq = (M & kSQ) ? get_u64(&pp->sq) : 0ull;
            const unsigned long long wsm = (M & kSMIN) ? get_u64(&pp->smin) : 0ull;
            const unsigned long long wam = (M & kAM) ? get_u64(&pp->am) : 0ull;
            const bool ok = f64_ok(wsp, ep) && (!(M & kSQ) || f64_ok(wsq, ep)) && (!(M & kSMIN) || f64_ok(wsm, ep)) &&
                            (!(M & kAM) || am_ok(wam, ep));
            if (ok && !a.force_recompute) {
                f.sp[e] = f64_of(wsp);
                f.sq[e] = f64_of(wsq);
                f.smin[e] = f64_of(wsm);
                f.am[e] = wam;
                need[j] = false;
            } else {
                any = true;
            }
        }
        if (!__syncthreads_or(any)) return;   // everything arrived (the usual case)
        if (wait_expired(a, t0)) break;
        __builtin_amdgcn_s_sleep(2);
    }
    // what is still missing (rare): recompute it, one entry at a time
    __shared__ int s_e;
    for (int e0 = 0; e0 < n_ent; ++e0) {
        bool mine = false;
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            if (need[j] && (int)threadIdx.x + j * kThreads == e0) mine = true;
        if (!__syncthreads_or(mine)) continue;
        if (mine) s_e = e0;
        __syncthreads();
        const int e = s_e, r = e / NC, c = e - r * NC, i = row0 + r;
        const int64_t row = (int64_t)b * (K + 1) + i;
        const Row prow = row_of(a.tp + row * V, V);
        const Row qrow = i < K ? row_of(a.dp + ((int64_t)b * K + i) * V, V) : prow;
        const Acc st = i < K ? block_reduce<MROW>(thread_stats_reload<VEC, MROW, kVecS>(prow, qrow, c))
                             : block_reduce<MLAST>(thread_stats_reload<VEC, MLAST, kVecS>(prow, prow, c));
        if (threadIdx.x == 0) {
            f.sp[e] = strip8(st.sp);
            f.sq[e] = strip8(st.sq);
            f.smin[e] = strip8(st.smin);
            f.am[e] = tag_am(st.maxv, st.arg, a.epoch);
            put_u32(&a.hdr->slow_path, 1u);
        }
        __syncthreads();
    }
}

// Wave-cooperative combine of the tile row whose entries start at `base`
// (the order of combine_row; values valid in every lane).
template <int M>
__device__ __forceinline__ RowView combine_flat(const FlatGathered& f, int base, int NC)
{
    const int lane = threadIdx.x & 63;
    RowView v{0.0, 0.0, 0.0, -INFINITY, INT_MAX};
    v.P = sum_chunks(&f.sp[base], NC);
    if constexpr ((M & kSQ) != 0) v.Q = sum_chunks(&f.sq[base], NC);
    if constexpr ((M & kSMIN) != 0) v.Smin = sum_chunks(&f.smin[base], NC);
    if constexpr ((M & kAM) != 0) {
        float mv = -INFINITY;
        int ai = INT_MAX;
        for (int h = 0; h < 2; ++h) {
            const int c = lane + 64 * h;
            if (c < NC) argmax_merge(mv, ai, am_val(f.am[base + c]), am_arg(f.am[base + c]));
        }
        wave_argmax(mv, ai);
        v.maxv = mv;
        v.arg = ai;
    }
    return v;
}

// Block-cooperative: the row statistics of every row of sequence b, written
// by the block that finishes it.  Rows go in tiles of as many rows as the
// LDS tile holds (all of them for K + 1 <= 512 / NC): thread t loads the
// draft token of tile row t while the tile's partials are gathered, then
// that token's values while the waves combine the rows (wave w takes rows w,
// w + 4, ...), and writes row t's statistics.
template <bool VEC, int MROW, int MLAST>
__device__ void write_all_stats(const Args& a, int b)
{
    constexpr int kTileMax = 64;
    __shared__ RowView s_rv[kTileMax];
    const int NC = a.NC, K = a.K, V = a.V;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int per_tile = FlatGathered::kCap / NC < kTileMax ? FlatGathered::kCap / NC : kTileMax;
    for (int r0 = 0; r0 <= K; r0 += per_tile) {
        const int T = (K + 1 - r0) < per_tile ? (K + 1 - r0) : per_tile;
        const int i = r0 + t;
        const int64_t row = (int64_t)b * (K + 1) + i;
        int tk = -1;
        if (t < T && i < K) tk = a.dt[(int64_t)b * K + i];
        gather_flat<VEC, MROW, MLAST>(lds.f, a, b, r0, T);
        const bool tin = t < T && i < K && tk >= 0 && tk < V;
        const float pt = tin ? a.tp[row * V + tk] : 0.0f;
        const float qt = tin ? a.dp[((int64_t)b * K + i) * V + tk] : 0.0f;
        for (int r = w; r < T; r += kWaves) {
            const RowView rv = r0 + r < K ? combine_flat<MROW>(lds.f, r * NC, NC) : combine_flat<MLAST>(lds.f, r * NC, NC);
            if (lane == 0) s_rv[r] = rv;
        }
        __syncthreads();
        if (t < T) write_stats(a, row, s_rv[t], i < K, pt, qt, i < K);
        __syncthreads();
    }
}

// ----------------------------------------------------------- greedy --

template <bool VEC, bool STATS>
__global__ __launch_bounds__(kThreads) void sv_greedy_kernel(Args a)
{
    constexpr int M = STATS ? (kSP | kAM) : kAM;
    const int NC = a.NC, K = a.K, V = a.V;
    // one block per (sequence b, row r, chunk c): the shortest blocks, so
    // the grid ends without a long tail
    const unsigned w = blockIdx.x / (unsigned)NC;
    const int b = (int)(w / (unsigned)(K + 1));
    const int r = (int)(w - (unsigned)b * (unsigned)(K + 1));
    const int c = (int)(blockIdx.x - w * (unsigned)NC);
    const int64_t row = (int64_t)b * (K + 1) + r;
    float4 x[kVecG];
    load_chunk<VEC, kVecG>(row_of(a.tp + row * V, V), c, x);
    publish_part<M>(a, row, c, block_reduce<M, false>(thread_stats<M, kVecG>(x, x, c), 0));
    if (c != finisher_column(b, NC) || r != K) return;

    const Outcome o = finish_rows<VEC, false, kVecG, M, M>(lds_greedy, a, b, a.stats != nullptr);
    if (threadIdx.x == 0) {
        a.n_out[b] = o.n;
        a.next_out[b] = o.arg;
    }
}

// ---------------------------------------------------------- sampled --

// The mass partials (sum p, sum q) of one chunk of a row, as loaded by
// thread t < NC for chunk t, and (thread 0) the inputs of the row's
// acceptance test.
struct Poll {
    unsigned long long sp, sq;
    float pt, qt, u;
};


// All polled values at once: their loads are then all issued before the
// first wait, and waited for together.
__device__ __forceinline__ void settle_poll(Poll& p)
{
    settle(p.sp);
    settle(p.sq);
    settle(p.pt);
    settle(p.qt);
    settle(p.u);
}

__device__ __forceinline__ Poll poll_issue(const Args& a, int b, int i, int tok)
{
    Poll p{0ull, 0ull, 0.0f, 0.0f, 0.0f};
    const int t = threadIdx.x, K = a.K, V = a.V;
    const int64_t row = (int64_t)b * (K + 1) + i;
    if (t < a.NC && t < 64) {   // chunk t in lane t of wave 0 (poll_decide polls t + 64)
        const Part* pp = a.parts + row * a.NC + t;
        p.sp = get_u64(&pp->sp);
        p.sq = get_u64(&pp->sq);
    }
    if (t == 0) {
        const bool tin = tok >= 0 && tok < V;
        p.pt = tin ? a.tp[row * V + tok] : 0.0f;
        p.qt = tin ? a.dp[((int64_t)b * K + i) * V + tok] : 0.0f;
        p.u = a.u[row];
    }
    return p;
}

// Block-cooperative: the masses of row i from the polled partials
// (re-polling the ones that do not carry this call's tag yet) and the
// acceptance of its draft token.  Returns 0 (accepted), 1 (rejected), or -1
// when some partial is still missing at the wait bound.  Uniform result.
__device__ int poll_decide(const Args& a, int b, int i, Poll pl, double* P, double* Q)
{
    __shared__ double s_PQ[2];
    __shared__ int s_rej;
    const int NC = a.NC, t = threadIdx.x;
    const unsigned ep = a.epoch;
    const int64_t row = (int64_t)b * (a.K + 1) + i;
    // Wave 0 decides alone: lane t holds chunks t (polled by poll_issue) and
    // t + 64 (polled here, rows of more than 64 chunks only); tags are
    // checked by ballot and the sums are those of sum_chunks, in registers.
    // One barrier then hands the result to the block.
    if (t < 64) {
        const Part* p0 = a.parts + row * NC + t;
        const Part* p1 = p0 + 64;
        bool need0 = t < NC, need1 = t + 64 < NC;
        unsigned long long w1p = 0ull, w1q = 0ull;
        if (need1) {
            w1p = get_u64(&p1->sp);
            w1q = get_u64(&p1->sq);
        }
        double s0p = 0.0, s0q = 0.0, s1p = 0.0, s1q = 0.0;
        const unsigned long long t0 = wall_clock64();
        for (;;) {
            if (need0 && f64_ok(pl.sp, ep) && f64_ok(pl.sq, ep) && !a.force_recompute) {
                s0p = f64_of(pl.sp);
                s0q = f64_of(pl.sq);
                need0 = false;
            }
            if (need1 && f64_ok(w1p, ep) && f64_ok(w1q, ep) && !a.force_recompute) {
                s1p = f64_of(w1p);
                s1q = f64_of(w1q);
                need1 = false;
            }
            if (__ballot(need0 || need1) == 0ull) break;
            if (a.force_recompute || wall_clock64() - t0 > a.poll_ticks) break;
            __builtin_amdgcn_s_sleep(2);
            if (need0) {
                pl.sp = get_u64(&p0->sp);
                pl.sq = get_u64(&p0->sq);
            }
            if (need1) {
                w1p = get_u64(&p1->sp);
                w1q = get_u64(&p1->sq);
            }
        }
        if (__ballot(need0 || need1) == 0ull && !a.force_lost) {
            const double p = wave_sum(s0p + s1p), q = wave_sum(s0q + s1q);
            if (t == 0) {
                s_PQ[0] = p;
                s_PQ[1] = q;
                s_rej = accepted(pl.u, pl.pt, pl.qt, p, q) ? 0 : 1;
            }
        } else if (t == 0) {
            s_rej = -1;
        }
    }
    __syncthreads();
    *P = s_PQ[0];
    *Q = s_PQ[1];
    return s_rej;
}

// Park this thread's share of a row chunk in LDS, and the residual sum of
// the parked share.
__device__ __forceinline__ void park(const float4 (&xp)[kVecS], const float4 (&xq)[kVecS])
{
#pragma unroll
    for (int k = 0; k < kVecS; ++k) {
        lds.parked[k][threadIdx.x] = f32x4{xp[k].x, xp[k].y, xp[k].z, xp[k].w};
        lds.parked[kVecS + k][threadIdx.x] = f32x4{xq[k].x, xq[k].y, xq[k].z, xq[k].w};
    }
}

// The order is that of thread_resid_reload (k ascending, one float4 each).
__device__ __forceinline__ double parked_resid(double P, double Q)
{
    double w = 0.0;
#pragma unroll
    for (int k = 0; k < kVecS; ++k) {
        const f32x4 p = lds.parked[k][threadIdx.x], q = lds.parked[kVecS + k][threadIdx.x];
        w += resid_f4(make_float4(p.x, p.y, p.z, p.w), make_float4(q.x, q.y, q.z, q.w), P, Q);
    }
    return w;
}

// Block-cooperative: the residual chunk masses of row n (published by the
// walking blocks) into m[0..NC); missing ones, and ones published as NaN
// (their block could not decide), are recomputed.
template <bool VEC>
__device__ void gather_resid(const Args& a, int b, int n, double P, double Q, double* m)
{
    __shared__ unsigned long long s_miss[2];
    const int NC = a.NC, K = a.K, V = a.V;
    const unsigned ep = a.epoch;
    const unsigned long long* wp = a.wpart + ((int64_t)b * K + n) * NC;
    const int c = threadIdx.x;
    bool need = c < NC, redo = false;
    const unsigned long long t0 = wall_clock64();
    for (;;) {
        bool any = false;
        if (need) {
            const unsigned long long wv = get_u64(&wp[c]);
            if (f64_ok(wv, ep) && !a.force_recompute) {
                m[c] = f64_of(wv);
                need = false;
                if (m[c] != m[c]) redo = true;   // published as "recompute"
            } else {
                any = true;
            }
        }
        if (!__syncthreads_or(any)) break;
        if (wait_expired(a, t0)) break;
        __builtin_amdgcn_s_sleep(2);
    }
    if (!__syncthreads_or(need || redo)) return;   // everything arrived (the usual case)
    if (threadIdx.x < 2) s_miss[threadIdx.x] = 0ull;
    __syncthreads();
    if (need || redo) atomicOr(&s_miss[c >> 6], 1ull << (c & 63));   // LDS
    __syncthreads();
    const Row prow = row_of(a.tp + ((int64_t)b * (K + 1) + n) * V, V);
    const Row qrow = row_of(a.dp + ((int64_t)b * K + n) * V, V);
    for (int h = 0; h < 2; ++h) {
        unsigned long long mk = s_miss[h];
        while (mk) {
            const int cc = h * 64 + __ffsll((unsigned long long)mk) - 1;
            mk &= mk - 1;
            const double w = block_sum(thread_resid_reload<VEC, kVecS>(prow, qrow, cc, P, Q));
            if (threadIdx.x == 0) {
                m[cc] = strip8(w);
                put_u32(&a.hdr->slow_path, 1u);
            }
        }
    }
    __syncthreads();
}

// Search state of a walking block (the same in every block of a sequence,
// since every block takes the same decisions from the same masses).
enum : int { kSearching = -1, kLost = -2 };

// Block-cooperative: the final draw of sequence b once its accept-prefix
// length n and the masses of row n are known, and the outputs.  n < K: the
// inverse CDF of the residual of row n, located by the published residual
// chunk masses; n == K (or, by rounding only, a rejection that left no
// residual mass): the inverse CDF of p_n, located by its target chunk masses.
template <bool VEC, int MB>
__device__ void draw_and_write(const Args& a, int b, int n, double Pn, double Qn)
{
    __shared__ double s_m[kMaxNC];
    __shared__ int s_owner, s_resid;
    __shared__ double s_base, s_T;
    const int NC = a.NC, K = a.K, V = a.V;
    const int64_t row0 = (int64_t)b * (K + 1);
    const double uK = (double)a.u[row0 + K];
    const Row prow = row_of(a.tp + (row0 + n) * V, V);
    const Row qrow = n < K ? row_of(a.dp + ((int64_t)b * K + n) * V, V) : prow;
    if (n < K) gather_resid<VEC>(a, b, n, Pn, Qn, s_m);
    if (threadIdx.x < 64) {
        int owner = -1;
        double base = 0.0, T = 0.0, W = 0.0;
        if (n < K) W = locate_chunk(s_m, NC, uK, &owner, &base, &T);
        if (threadIdx.x == 0) {
            s_owner = owner;
            s_base = base;
            s_T = T;
            s_resid = (n < K && W > 0.0) ? 1 : 0;
        }
    }
    __syncthreads();
    if (!s_resid) {
        if (n < K)
            gather_rows<VEC, kVecS, kSP, kSP>(lds.g, a, b, n, 1);
        else
            gather_rows<VEC, kVecS, kSP, MB>(lds.g, a, b, n, 1);
        if (threadIdx.x < 64) {
            int owner;
            double base, T;
            locate_chunk(lds.g.sp[0], NC, uK, &owner, &base, &T);
            if (threadIdx.x == 0) {
                s_owner = owner;
                s_base = base;
                s_T = T;
            }
        }
        __syncthreads();
    }
    int x = -1;
    if (s_owner >= 0)
        x = s_resid ? chunk_draw<VEC, true, kVecS>(prow, qrow, Pn, Qn, s_owner, s_base, s_T)
                    : chunk_draw<VEC, false, kVecS>(prow, prow, Pn, Qn, s_owner, s_base, s_T);
    if (threadIdx.x == 0) {
        a.n_out[b] = n;
        a.next_out[b] = x;
    }
    __syncthreads();
}

// The outcome a sequence's finishing walk publishes for the block that
// finishes its bonus row: n + 1 once n is known (the draw is then already
// made when n < K), 0 when the walk could not decide; tagged like every
// published word.
__device__ __forceinline__ unsigned long long tag_state(int code, unsigned ep)
{
    return ((unsigned long long)(unsigned)code << 8) | ep;
}

// Block-cooperative: the finishing step of sequence b, run by the block of
// its bonus row that finishes it (the last work of the sequence).
template <bool VEC, bool STATS, bool ROWS>
__device__ __forceinline__ void finish_bonus(const Args& a, int b)
{
    constexpr int MP = STATS ? (kSP | kSQ | kSMIN | kAM) : (kSP | kSQ);
    constexpr int MB = STATS ? (kSP | kAM) : kSP;
    __shared__ int s_code;
    const int K = a.K;
    int n = -1;
    bool drawn = false;
    double Pn = 0.0, Qn = 0.0;
    if (K == 0) {
        n = 0;
    } else if (!ROWS) {
        // the walks' outcome (published when the walks ended, normally long
        // before this block runs); without it, decide here from the partials,
        // as always when each draft row has blocks of its own (no outcome)
        const unsigned long long t0 = wall_clock64();
        for (;;) {
            bool got = false;
            if (threadIdx.x == 0) {
                const unsigned long long v = get_u64(&a.sstate[b]);
                got = f64_ok(v, a.epoch) && !a.force_recompute;
                const unsigned long long code = v >> 8;
                s_code = got && code <= (unsigned long long)(K + 1) ? (int)code : 0;   // 0: decide here
            }
            if (__syncthreads_or(got)) break;
            if (wait_expired(a, t0)) break;
            __builtin_amdgcn_s_sleep(2);
        }
        const int code = s_code;
        __syncthreads();
        if (code > 0) {
            n = code - 1;
            drawn = n < K;
        }
    }
    if ((STATS && ROWS) || n < 0) {
        const Outcome o = finish_rows<VEC, true, kVecS, MP, MB>(lds.g, a, b, STATS && ROWS);
        n = o.n;
        Pn = o.P;
        Qn = o.Q;
    }
    // with statistics, the walks' finishing block writes every row's in tiles
    if (STATS && !ROWS) write_all_stats<VEC, MP, MB>(a, b);
    if (!drawn) draw_and_write<VEC, MB>(a, b, n, Pn, Qn);
}

// The same, not inlined: with row statistics the combine of every row adds
// enough code that, inlined, it would push the walk loop into spilling.  The
// callee reads the arguments where the kernel received them.
template <bool VEC, bool STATS, bool ROWS>
__device__ __noinline__ void finish_bonus_call(const Args& a, int b)
{
    finish_bonus<VEC, STATS, ROWS>(a, b);
}

template <bool VEC, bool STATS, bool ROWS, bool EARLY = false>
__global__ __launch_bounds__(kThreads, 4) void sv_sample_kernel(Args a)
{
    constexpr int MP = STATS ? (kSP | kSQ | kSMIN | kAM) : (kSP | kSQ);   // rows 0..K-1
    constexpr int MB = STATS ? (kSP | kAM) : kSP;                        // bonus row K
    const int NC = a.NC, K = a.K, V = a.V;

    if (blockIdx.x >= a.nwalk) {
        // Bonus row K (target only), one chunk per block.  These blocks come
        // after every walk in the grid: they are short, so they keep the
        // machine busy while the last walks end.  The block of the rotating
        // finishing column finishes the sequence.
        const int per_seq = (NC + kBonusChunks - 1) / kBonusChunks;
        const unsigned blk = blockIdx.x - a.nwalk;
        const int b = (int)(blk / (unsigned)per_seq);
        const int c0 = (int)(blk - (unsigned)b * (unsigned)per_seq) * kBonusChunks;
        const int64_t row0 = (int64_t)b * (K + 1);
        if (!ROWS && a.early && K > 0) {
            // Early exit: the bonus row is needed only after full acceptance.
            // Once the walks' outcome shows a rejection (they published it
            // when they ended, normally long before this block runs), nothing
            // reads this row.  Without the outcome the row is read as always.
            __shared__ int s_skip;
            if (threadIdx.x == 0) {
                const unsigned long long v = get_u64(&a.sstate[b]);
                const unsigned long long code = v >> 8;
                s_skip = f64_ok(v, a.epoch) && !a.force_recompute && code >= 1 && code <= (unsigned long long)K;
            }
            __syncthreads();
            if (s_skip) return;
        }
        const Row prow = row_of(a.tp + (row0 + K) * V, V);
        float4 xp[kBonusChunks][kVecS];
#pragma unroll
        for (int j = 0; j < kBonusChunks; ++j)   // chunks past NC read as zeros
            load_chunk_keep<VEC, kVecS>(prow, c0 + j < NC ? c0 + j : NC, xp[j], blk + kTailBlocks >= gridDim.x - a.nwalk);
#pragma unroll
        for (int j = 0; j < kBonusChunks; ++j)
            if (c0 + j < NC)
                publish_part<MB>(a, row0 + K, c0 + j, block_reduce<MB, false>(thread_stats<MB, kVecS>(xp[j], xp[j], c0 + j), j & 1));
        const int fc = finisher_column(b, NC);
        if (fc < c0 || fc >= c0 + kBonusChunks) return;
        __builtin_amdgcn_s_setprio(3);   // latency matters here: the last of these end the kernel
        if constexpr (STATS)
            finish_bonus_call<VEC, STATS, ROWS>(*(const Args*)(const void*)__builtin_amdgcn_kernarg_segment_ptr(), b);
        else
            finish_bonus<VEC, STATS, ROWS>(a, b);
        return;
    }

    if constexpr (ROWS) {
        // One block per (sequence b, draft row i, chunk c), every row at
        // once: the form for small grids, where a walk's row-after-row
        // latency would dominate.
        // The block publishes its partials, decides row i from its siblings'
        // (the decision every reader takes) and, when row i is rejected,
        // publishes its chunk's residual mass.  The block that finishes the
        // bonus row decides the sequence from the partials and draws.
        const unsigned w = blockIdx.x / (unsigned)NC;
        const int b = (int)(w / (unsigned)K);
        const int i = (int)(w - (unsigned)b * (unsigned)K);
        const int c = (int)(blockIdx.x - w * (unsigned)NC);
        const int64_t row = (int64_t)b * (K + 1) + i;
        float4 xp[kVecS], xq[kVecS];
        load_chunk<VEC, kVecS>(row_of(a.tp + row * V, V), c, xp);
        load_chunk<VEC, kVecS>(row_of(a.dp + ((int64_t)b * K + i) * V, V), c, xq);
        const int tok = threadIdx.x == 0 ? a.dt[(int64_t)b * K + i] : -1;
        publish_part<MP>(a, row, c, block_reduce<MP, false>(thread_stats<MP, kVecS>(xp, xq, c), 0));
        park(xp, xq);
        double P, Q;
        Poll pl = poll_issue(a, b, i, tok);
        settle_poll(pl);
        const int rej = poll_decide(a, b, i, pl, &P, &Q);
        if (rej != 0) {   // rejected: the residual mass; undecided: marked for recomputing
            const double m = rej > 0 ? block_sum(parked_resid(P, Q)) : __builtin_nan("");
            if (threadIdx.x == 0) put_u64(&a.wpart[((int64_t)b * K + i) * NC + c], tag_f64(m, a.epoch));
        }
        return;
    }

    // A walk: chunk column c of draft rows 0..K-1 of sequence b (K >= 1).
    const int b = (int)(blockIdx.x / (unsigned)NC);
    const int c = (int)(blockIdx.x - (unsigned)b * (unsigned)NC);
    const float* tb = a.tp + (int64_t)b * (K + 1) * V;
    const float* db = a.dp + (int64_t)b * K * V;
    const int64_t row0 = (int64_t)b * (K + 1);

    // At step i row i is in registers (xp, xq) and row i+1 loads into
    // (yp, yq).  While no draft has been rejected yet, row i-1 waits in LDS
    // for its decision: its partials were published by the sibling walks a
    // step ago and are polled (with the inputs of its acceptance test)
    // before row i+1's loads are issued, so, loads returning in order, they
    // arrive while those loads are in flight.  The first rejected row n gets
    // its chunk's residual mass published; after it the walk only streams.
    int state = kSearching;                // kSearching, kLost, or the decided n
    double Pn = 0.0, Qn = 0.0;
    int tok = -1;                          // draft token of the pending row (thread 0)
    float4 xp[kVecS], xq[kVecS], yp[kVecS], yq[kVecS];
    // While it searches, a walk's waves issue before those of walks that
    // only stream (priority 2 of 0..3; the finishing block takes 3): the
    // searching walks of a sequence move in step with their slowest sibling,
    // so they, not the streaming ones, decide when the last walks end.
    // Measured: 174.1 -> 171.8 us at B=32 K=16 V=262144, 1305.5 -> 1298.4 us
    // at B=1024 K=8 V=128256, 214.9 -> 214.6 us at B=256 K=5 V=128256.
    __builtin_amdgcn_s_setprio(2);
    load_chunk<VEC, kVecS>(row_of(tb, V), c, xp);
    load_chunk<VEC, kVecS>(row_of(db, V), c, xq);

    // decide row j (parked) from its poll; publish its residual if rejected
    auto decide = [&](int j, const Poll& pl) {
        double P, Q;
        const int rej = poll_decide(a, b, j, pl, &P, &Q);
        if (rej < 0) {
            // masses missing: leave the decision to the finisher, marking the
            // residuals of every row from j on as "recompute"
            state = kLost;
            if (threadIdx.x == 0)
                for (int r = j; r < K; ++r)
                    put_u64(&a.wpart[((int64_t)b * K + r) * NC + c], tag_f64(__builtin_nan(""), a.epoch));
        } else if (rej) {
            state = j;
            Pn = P;
            Qn = Q;
            const double w = block_sum(parked_resid(P, Q));
            if (threadIdx.x == 0) put_u64(&a.wpart[((int64_t)b * K + j) * NC + c], tag_f64(w, a.epoch));
        }
    };
    // row i+1's loads (an empty range after the last draft row reads zeros)
    auto load_next = [&](int i) {
        const bool more = i + 1 < K;
        const int64_t off = more ? (int64_t)(i + 1) * V : 0;
        load_chunk<VEC, kVecS>(row_of(tb + off, more ? V : 0), c, yp);
        load_chunk<VEC, kVecS>(row_of(db + off, more ? V : 0), c, yq);
    };

    int i = 0;
    if constexpr (STATS) {
        // With statistics, step 0 (no decision pending yet) runs before the
        // loop, so that where the loop reads (xp, xq) they always hold a
        // copied row, never one still loading: the compiler then has no
        // reason to wait there for the step's polls, issued just before the
        // next row's loads, and the longer reduction of the statistics
        // overlaps them (measured: 236.7 against 240.1 us at B=256 K=5
        // V=128256; without statistics the same form measured 217.5 against
        // 214.6 us, so that pass keeps the plain loop).
        if (threadIdx.x == 0) tok = a.dt[(int64_t)b * K];   // row 0's token, for step 1
        __builtin_amdgcn_sched_barrier(0);
        if (!EARLY) load_next(0);
        __builtin_amdgcn_sched_barrier(0);
        publish_part<MP>(a, row0, c, block_reduce<MP, false>(thread_stats<MP, kVecS>(xp, xq, c), 0));
        if (EARLY) load_next(0);
        park(xp, xq);
#pragma unroll
        for (int k = 0; k < kVecS; ++k) {
            xp[k] = yp[k];
            xq[k] = yq[k];
        }
        // row 1 has arrived (the copy needs it anyway); the explicit wait
        // tells the compiler so, which could otherwise hand row 1's load
        // registers to the loop as still loading
        __builtin_amdgcn_s_waitcnt(0);
        i = 1;
    }
    for (; i < K; ++i) {   // searching: decisions one step behind, rows parked
        Poll pl{0ull, 0ull, 0.0f, 0.0f, 0.0f};
        const bool pending = STATS || i > 0;
        if (pending) pl = poll_issue(a, b, i - 1, tok);
        if (threadIdx.x == 0) tok = a.dt[(int64_t)b * K + i];   // row i's token, for step i+1
        __builtin_amdgcn_sched_barrier(0);
        if (!EARLY) load_next(i);
        __builtin_amdgcn_sched_barrier(0);
        // the polls are settled (waited for) after the reduction and before
        // the partials are stored (a store issued after the row loads would
        // make that wait cover some of them)
        const Acc r = block_reduce<MP, false>(thread_stats<MP, kVecS>(xp, xq, c), i & 1);
        if (pending) settle_poll(pl);
        publish_part<MP>(a, row0 + i, c, r);
        if (pending) decide(i - 1, pl);
        // the early exit issues row i+1's loads only once row i-1 is
        // accepted (or its decision is lost: the walk then still streams
        // every row), so that a rejection at n leaves rows n+2.. unread
        if (EARLY && state < 0) load_next(i);
        if (state == kSearching) park(xp, xq);
#pragma unroll
        for (int k = 0; k < kVecS; ++k) {
            xp[k] = yp[k];
            xq[k] = yq[k];
        }
        if (state != kSearching) {
            ++i;
            break;
        }
    }
    // Early exit: after a decided rejection no later row is read.  Every
    // reader of this sequence needs rows 0..n only (the decisions, the
    // residual of row n); the row after n is already in flight.  A walk
    // that lost its decision still publishes every row, for the finisher.
    if (EARLY && state >= 0) i = K;
    __builtin_amdgcn_s_setprio(0);   // searching is over: back to the default priority
    for (; i < K; ++i) {   // after the first rejection (or a lost decision)
        load_next(i);
        __builtin_amdgcn_sched_barrier(0);
        publish_part<MP>(a, row0 + i, c, block_reduce<MP, false>(thread_stats<MP, kVecS>(xp, xq, c), i & 1));
#pragma unroll
        for (int k = 0; k < kVecS; ++k) {
            xp[k] = yp[k];
            xq[k] = yq[k];
        }
    }
    if (state == kSearching) {   // the last draft row's decision
        Poll pl = poll_issue(a, b, K - 1, tok);
        settle_poll(pl);
        decide(K - 1, pl);
        if (state == kSearching) state = K;   // every draft accepted
    }
    if (c != finisher_column(b, NC)) return;

    // The finishing walk of sequence b draws when a draft was rejected and
    // publishes the outcome for the block that finishes the bonus row.
    __builtin_amdgcn_s_setprio(3);
    if (state >= 0 && state < K) draw_and_write<VEC, MB>(a, b, state, Pn, Qn);
    if (threadIdx.x == 0) put_u64(&a.sstate[b], tag_state(state >= 0 ? state + 1 : 0, a.epoch));
}

// ------------------------------------------------------------ logits --
//
// Sampled verification on logits warped by a temperature tau.  The warped
// distribution of a row of logits l is softmax(l / tau); the card asks that
// target and draft be warped identically, and one tau warps both here.  The
// work decomposition, the walk and the finishing are those of
// sv_sample_kernel; what a chunk publishes differs.  Per operand, a chunk
// publishes its maximum m_c (positions at or past V left out) and the sum s_c
// of the weights exp((l - m_c) / tau) = exp2((l - m_c) * k), k = log2(e) /
// tau: each wave sums its values' weights against its own maximum (per
// thread in fp32, then across the wave in fp64), and the chunk rescales the
// four wave sums to m_c in wave order.  A reader of a row takes its maximum M
// (the largest m_c) and its mass sum_c s_c exp2((m_c - M) * k), in chunk
// order (chunk_scaled).  Single weights (the residual, the draws) are
// exp2((l - M) * k) against the same M, on the scale of that mass; the two
// weights of an acceptance test take more care over range and rounding
// (accepted_l).

// The weight of a logit l against a maximum m: exp2(l * k - r) with
// r = m * k rounded to fp32, the argument one fused multiply-add (l * k
// exact inside it).  Every weight taken against the same m shares the one
// rounding of r; weights taken against different maxima are brought to a
// common one by chunk_scaled, which uses the same rounded products, so the
// rounding cancels there too.
__device__ __forceinline__ float lweight(float l, float m, float k)
{
    return __builtin_amdgcn_exp2f(__builtin_fmaf(l, k, -(m * k)));
}

// The weight of a draft token's logit for its acceptance test, with fp64
// range and an fp64 temperature.  At a low temperature a token far from its
// row's maximum has an exponent far below fp32's range (-650 for a logit 9
// below the maximum at tau 0.02): in fp32 both of its weights would flush to
// zero and decide 0 < 0, whatever the ratio p(t)/q(t) they stand for; and
// the fp32 k = log2(e) / tau, exact to 6e-8 relative, would move an exponent
// of -650 by 4e-5.  The exponent here is (l - m) * k64 plus the rounding
// m * k - r of the row's shared scale r = m * k (fp32): the row mass carries
// the factor 2^(m k - r) in every weight, so it still cancels in the test.
// It splits exactly into n = floor(e) and f = e - n in [0, 1), and the weight
// is 2^f (fp32, f rounded by at most 2^-25) scaled by 2^n in fp64: about
// 1.5e-7 relative in all.  -inf logits give 0.
__device__ __forceinline__ double lweight_wide(float l, float m, float k, double k64)
{
    const float r = m * k;
    const double e = __builtin_fma((double)l - (double)m, k64, __builtin_fma((double)m, (double)k, -(double)r));
    if (!(e > -1100.0)) return e != e ? e : 0.0;   // NaN stays NaN (rejects); below fp64's range, 0
    const double n = __builtin_floor(e);
    return __builtin_ldexp((double)__builtin_amdgcn_exp2f((float)(e - n)), (int)n);
}

// Maximum over the wave (all 64 lanes active), the same in every lane.
__device__ __forceinline__ float wave_maxf(float v)
{
    v = fmaxf(v, __int_as_float(dpp_i32<kDppPairs>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_i32<kDppQuads>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_i32<kDppHalfMirror>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_i32<kDppMirror>(__float_as_int(v))));
    unsigned a, b;   // the row maxima as max(max(r0, r1), max(r2, r3)), as wave_sum orders its sums
    rows_01_23(__float_as_uint(v), a, b);
    halves(__float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b))), a, b);
    return fmaxf(__uint_as_float(a), __uint_as_float(b));
}

// Whether every position of chunk c lies below V (no masking needed).
template <int NV>
__device__ __forceinline__ bool chunk_full(int c, int V)
{
    return (int64_t)(c + 1) * (kThreads * NV * 4) <= (int64_t)V;
}

// Set the positions of chunk c at or past V to -inf: such a value cannot be
// a maximum and its weight exp2(-inf) is +0, which leaves every sum as it
// would be without the position.  Only the ragged last chunk of a row has
// such positions; the empty asm keeps this on a branch of its own, so a
// full chunk pays nothing for it.
template <int NV>
__device__ __forceinline__ void mask_tail_l(float4 (&v)[NV], int c, int V)
{
    if (chunk_full<NV>(c, V)) return;
    asm volatile("");
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int p0 = 4 * f4_index<NV>(c, k);
        if (p0 >= V) v[k].x = -INFINITY;
        if (p0 + 1 >= V) v[k].y = -INFINITY;
        if (p0 + 2 >= V) v[k].z = -INFINITY;
        if (p0 + 3 >= V) v[k].w = -INFINITY;
    }
}

// Largest value of the thread's share (-inf if it holds no position < V).
template <int NV>
__device__ __forceinline__ float share_max(const float4 (&v)[NV])
{
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < NV; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) m = fmaxf(m, comp(v[k], e));
    return m;
}

// Sum of the weights of the thread's share against m: its 4 * NV weights (at
// most 1 each) in fp32, k then e ascending, then fp64 from there on.  A
// share whose values are all -inf (m = -inf) sums to 0.
template <int NV>
__device__ __forceinline__ double share_wsum(const float4 (&v)[NV], float m, float k)
{
    const float nmk = m == -INFINITY ? 0.0f : -(m * k);   // the argument of lweight(l, m, k)
    // the first weight starts the sum (0 + w is w: a weight is never -0)
    float s = __builtin_amdgcn_exp2f(__builtin_fmaf(comp(v[0], 0), k, nmk));
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int e = (j == 0 ? 1 : 0); e < 4; ++e) s += __builtin_amdgcn_exp2f(__builtin_fmaf(comp(v[j], e), k, nmk));
    return (double)s;
}

// A chunk sum s of weights taken against maximum m, rescaled to reference M
// (0 for an empty chunk): s * exp2(r_m - r_M), r_x = x * k rounded to fp32 as
// in lweight.  The rounding of r_m in the chunk's weights cancels, and that
// of r_M is the one every weight against M carries.  The difference of the
// two products is exact when they lie within a factor of 2 of each other and
// otherwise rounded once, like any weight's own argument.  The exact m * k
// of an fma here instead would leave the rounding of r_m in every weight of
// the chunk: at tau = 0.02 (k = 72, |m * k| ~ 600) that is 2e-5 of the row's
// mass.
__device__ __forceinline__ double chunk_scaled(float m, double s, float M, float k)
{
    if (m == -INFINITY) return 0.0;
    const float rm = m * k, rM = M * k;   // not contracted: fp contract is off in this file
    return s * (double)__builtin_amdgcn_exp2f(rm - rM);
}

struct LStat {
    float mp, mq;      // chunk maxima (every thread)
    double sp, sq;     // weight sums against them (thread 0)
};

// Block-cooperative: (m_c, s_c) of target chunk pv and, with Q, of draft
// chunk qv, valid in thread 0.  Each wave sums its weights against its own
// maximum (found by DPP, no barrier); wave 0 takes the chunk maximum m_c
// over the four waves and rescales their sums to it, adding them in wave
// order.  The positions of pv and qv at or past V are set to -inf
// (mask_tail_l).  Consecutive calls alternate `slot`, as for block_reduce.
template <int NV, bool Q>
__device__ __forceinline__ LStat chunk_stats_l(float4 (&pv)[NV], float4 (&qv)[NV], int c, int V, float k, int slot)
{
    __shared__ float s_m[2][2][kWaves];
    __shared__ double s_s[2][2][kWaves];
    mask_tail_l<NV>(pv, c, V);
    if (Q) mask_tail_l<NV>(qv, c, V);
    const float mp = wave_maxf(share_max<NV>(pv));
    const double sp = wave_sum(share_wsum<NV>(pv, mp, k));
    float mq = -INFINITY;
    double sq = 0.0;
    if (Q) {
        mq = wave_maxf(share_max<NV>(qv));
        sq = wave_sum(share_wsum<NV>(qv, mq, k));
    }
    // the wave's LDS address formed here at every call (as in poll_issue_l):
    // kept for the whole walk it went to scratch, and its reload held every
    // step's reduction until that step's row loads had arrived
    // (234.8 -> 232.6 us at B=256 K=5 V=128256)
    int tid = threadIdx.x;
    settle(tid);
    const int lane = tid & 63, w = tid >> 6;
    if (lane == 0) {
        s_m[slot][0][w] = mp;
        s_s[slot][0][w] = sp;
        s_m[slot][1][w] = mq;
        s_s[slot][1][w] = sq;
    }
    __syncthreads();
    LStat r{mp, mq, 0.0, 0.0};
    if (tid < 64) {
        // Lane 4 o + j of wave 0 rescales wave j's sum of operand o (one
        // exp2 each, side by side rather than eight in a row on one lane);
        // the four terms of an operand are then added in wave order, the
        // sum one lane would form (230.9 against 232.0 us at B=256 K=5
        // V=128256).  Lanes 8..63 repeat lanes 0..7.
        static_assert(kWaves == 4, "one lane per (operand, wave) pair in a group of four");
        const int o = Q ? (lane >> 2) & 1 : 0, j = lane & 3, g = lane & ~3;
        float M = s_m[slot][o][0];
        for (int jj = 1; jj < kWaves; ++jj) M = fmaxf(M, s_m[slot][o][jj]);
        const double t = chunk_scaled(s_m[slot][o][j], s_s[slot][o][j], M, k);
        // lanes g+1..g+3 of the quad by DPP, lane 4's results by scalar reads
        const double t1 = dpp_f64<0x55>(t), t2 = dpp_f64<0xAA>(t), t3 = dpp_f64<0xFF>(t);
        const double S = ((t + t1) + t2) + t3;
        const unsigned long long sb = (unsigned long long)__double_as_longlong(S);
        const double Sq = __longlong_as_double(
            (long long)(((unsigned long long)(unsigned)__builtin_amdgcn_readlane((int)(sb >> 32), 4) << 32) |
                        (unsigned)__builtin_amdgcn_readlane((int)sb, 4)));
        const float Mq = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(M), 4));
        if (lane == 0) {
            r.mp = M;
            r.sp = S;
            if (Q) {
                r.mq = Mq;
                r.sq = Sq;
            }
        }
    }
    return r;
}

// Publish a chunk's (m, s): sums as tagged fp64 words (sp, sq), maxima as
// tagged (value, 0) words in the am (target) and smin (draft) slots.
__device__ __forceinline__ void publish_l(const Args& a, int64_t row, int c, const LStat& s, bool q)
{
    if (threadIdx.x == 0) {
        Part* dst = &a.parts[row * a.NC + c];
        put_u64(&dst->sp, tag_f64(s.sp, a.epoch));
        put_u64(&dst->am, tag_am(s.mp, 0, a.epoch));
        if (q) {
            put_u64(&dst->sq, tag_f64(s.sq, a.epoch));
            put_u64(&dst->smin, tag_am(s.mq, 0, a.epoch));
        }
    }
}

// Wave-cooperative: a row's maximum and mass from the chunks a lane holds
// (chunks l and l + 64; m = -inf for none): M is the largest m, the mass is
// sum_c s_c exp2((m_c - M) k), a lane's pair first, then the fixed wave sum.
// Every reader of a row uses this.
__device__ __forceinline__ double row_mass_l(float m0, double s0, float m1, double s1, float k, float* Mout)
{
    const float M = wave_maxf(fmaxf(m0, m1));
    *Mout = M;
    return wave_sum(chunk_scaled(m0, s0, M, k) + chunk_scaled(m1, s1, M, k));
}

// Residual mass of one position: max(0, w_p Q - w_q P), fp64.
__device__ __forceinline__ double resid_l(float lp, float lq, double P, double Q, float Mp, float Mq, float k)
{
    const double d = (double)lweight(lp, Mp, k) * Q - (double)lweight(lq, Mq, k) * P;
    return d > 0.0 ? d : 0.0;
}

struct LRow {
    double P, Q;
    float Mp, Mq;
};

// The acceptance test of a draft token on logits, for exponents outside
// [-16, 0]: the token weights with fp64 range and temperature (lweight_wide).
// Not inlined, so that its fp64 work adds nothing to the registers of the
// streaming loops it is reached from.  Everything it needs comes in as
// arguments: inside a called function the kernel-argument segment pointer
// is not available (the compiler materialises it as null).
__device__ __noinline__ bool accepted_wide_l(float u, float lp, float lq, float Mp, float Mq, double P, double Q,
                                             float k, double k64)
{
    return accepted(u, lweight_wide(lp, Mp, k, k64), lweight_wide(lq, Mq, k, k64), P, Q);
}

// The acceptance test of draft token logits lp = l_p(t), lq = l_q(t) against
// row r (tin: the token is inside [0, V); a token outside is rejected).
// Where both fp32 exponents lie in [-16, 0] the fp32 weights serve: the
// rounding of k (6e-8 relative) and of the exponents moves the ratio
// p(t)/q(t) by under 3e-6 there.  Elsewhere the fp64 test decides.  Every
// place that decides a logits row uses this function.
__device__ __forceinline__ bool accepted_l(bool tin, float u, float lp, float lq, const LRow& r, float k, double k64)
{
    if (!tin) return false;
    const float ap = __builtin_fmaf(lp, k, -(r.Mp * k));
    const float aq = __builtin_fmaf(lq, k, -(r.Mq * k));
    if (ap >= -16.0f && aq >= -16.0f)
        return accepted(u, __builtin_amdgcn_exp2f(ap), __builtin_amdgcn_exp2f(aq), r.P, r.Q);
    return accepted_wide_l(u, lp, lq, r.Mp, r.Mq, r.P, r.Q, k, k64);
}

// The walk's poll of row i: lane c < min(NC, 64) of wave 0 reads chunk c's
// four words; lane 0 also the logits at the draft token and the uniform.
struct PollL {
    unsigned long long sp, sq, mp, mq;
    float pt, qt, u;
    int tin;
};

__device__ __forceinline__ void settle_poll_l(PollL& p)
{
    settle(p.sp);
    settle(p.sq);
    settle(p.mp);
    settle(p.mq);
    settle(p.pt);
    settle(p.qt);
    settle(p.u);
    settle(p.tin);
}

__device__ __forceinline__ PollL poll_issue_l(const Args& a, int b, int i, int tok)
{
    PollL p{0ull, 0ull, 0ull, 0ull, 0.0f, 0.0f, 0.0f, 0};
    // The thread index passes through an empty asm so that the lane's word
    // address is formed here at every call: hoisted out of the walk, it was
    // one more value to keep for the whole walk, and at 128 VGPRs it went to
    // scratch, whose reload waited (in order) for the row loads in flight.
    int t = threadIdx.x;
    settle(t);
    const int K = a.K, V = a.V;
    const int64_t row = (int64_t)b * (K + 1) + i;
    if (t < a.NC && t < 64) {
        const Part* pp = a.parts + row * a.NC + t;
        p.sp = get_u64(&pp->sp);
        p.sq = get_u64(&pp->sq);
        p.mp = get_u64(&pp->am);
        p.mq = get_u64(&pp->smin);
    }
    if (t == 0) {
        p.tin = tok >= 0 && tok < V;
        p.pt = p.tin ? a.tp[row * V + tok] : 0.0f;
        p.qt = p.tin ? a.dp[((int64_t)b * K + i) * V + tok] : 0.0f;
        p.u = a.u[row];
    }
    return p;
}

__device__ __forceinline__ bool lwords_ok(unsigned long long sp, unsigned long long sq, unsigned long long mp,
                                          unsigned long long mq, unsigned ep)
{
    return f64_ok(sp, ep) && f64_ok(sq, ep) && am_ok(mp, ep) && am_ok(mq, ep);
}

// Block-cooperative (wave 0 decides, as in poll_decide): the masses and
// maxima of row i and the acceptance of its draft token.  Returns 0, 1, or
// -1 when some word is still missing at the wait bound.  Uniform result.
__device__ int poll_decide_l(const Args& a, int b, int i, PollL pl, LRow* out)
{
    __shared__ LRow s_row;
    __shared__ int s_rej;
    const int NC = a.NC;
    int t = threadIdx.x;
    settle(t);   // as in poll_issue_l: addresses formed here, not kept in scratch
    const unsigned ep = a.epoch;
    const float k = a.ktau;
    const int64_t row = (int64_t)b * (a.K + 1) + i;
    if (t < 64) {
        const Part* p0 = a.parts + row * NC + t;
        const Part* p1 = p0 + 64;
        bool need0 = t < NC, need1 = t + 64 < NC;
        unsigned long long w1[4] = {0ull, 0ull, 0ull, 0ull};
        if (need1) {
            w1[0] = get_u64(&p1->sp);
            w1[1] = get_u64(&p1->sq);
            w1[2] = get_u64(&p1->am);
            w1[3] = get_u64(&p1->smin);
        }
        float m0p = -INFINITY, m0q = -INFINITY, m1p = -INFINITY, m1q = -INFINITY;
        double s0p = 0.0, s0q = 0.0, s1p = 0.0, s1q = 0.0;
        const unsigned long long t0 = wall_clock64();
        for (;;) {
            if (need0 && lwords_ok(pl.sp, pl.sq, pl.mp, pl.mq, ep) && !a.force_recompute) {
                s0p = f64_of(pl.sp);
                s0q = f64_of(pl.sq);
                m0p = am_val(pl.mp);
                m0q = am_val(pl.mq);
                need0 = false;
            }
            if (need1 && lwords_ok(w1[0], w1[1], w1[2], w1[3], ep) && !a.force_recompute) {
                s1p = f64_of(w1[0]);
                s1q = f64_of(w1[1]);
                m1p = am_val(w1[2]);
                m1q = am_val(w1[3]);
                need1 = false;
            }
            if (__ballot(need0 || need1) == 0ull) break;
            if (a.force_recompute || wall_clock64() - t0 > a.poll_ticks) break;
            __builtin_amdgcn_s_sleep(2);
            if (need0) {
                pl.sp = get_u64(&p0->sp);
                pl.sq = get_u64(&p0->sq);
                pl.mp = get_u64(&p0->am);
                pl.mq = get_u64(&p0->smin);
            }
            if (need1) {
                w1[0] = get_u64(&p1->sp);
                w1[1] = get_u64(&p1->sq);
                w1[2] = get_u64(&p1->am);
                w1[3] = get_u64(&p1->smin);
            }
        }
        if (__ballot(need0 || need1) == 0ull && !a.force_lost) {
            LRow r;
            r.P = row_mass_l(m0p, s0p, m1p, s1p, k, &r.Mp);
            r.Q = row_mass_l(m0q, s0q, m1q, s1q, k, &r.Mq);
            if (t == 0) {
                s_row = r;
                s_rej = accepted_l(pl.tin, pl.u, pl.pt, pl.qt, r, k, a.ktau64) ? 0 : 1;
            }
        } else if (t == 0) {
            s_rej = -1;
        }
    }
    __syncthreads();
    *out = s_row;
    return s_rej;
}

// Residual mass of the thread's parked share (k, then e, ascending).
__device__ __forceinline__ double parked_resid_l(const LRow& r, float k, int c, int V)
{
    const bool full = chunk_full<kVecS>(c, V);
    double w = 0.0;
#pragma unroll
    for (int j = 0; j < kVecS; ++j) {
        const f32x4 p = lds.parked[j][threadIdx.x], q = lds.parked[kVecS + j][threadIdx.x];
        const int p0 = 4 * f4_index<kVecS>(c, j);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (full || p0 + e < V) w += resid_l(p[e], q[e], r.P, r.Q, r.Mp, r.Mq, k);
    }
    return w;
}

// The same sum re-reading the chunk (same order).
template <bool VEC>
__device__ __forceinline__ double thread_resid_reload_l(Row prow, Row qrow, int c, int V, const LRow& r, float k)
{
    const bool full = chunk_full<kVecS>(c, V);
    double w = 0.0;
    for (int j = 0; j < kVecS; ++j) {
        const float4 p4 = load_one<VEC, kVecS>(prow, c, j), q4 = load_one<VEC, kVecS>(qrow, c, j);
        const int p0 = 4 * f4_index<kVecS>(c, j);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (full || p0 + e < V) w += resid_l(comp(p4, e), comp(q4, e), r.P, r.Q, r.Mp, r.Mq, k);
    }
    return w;
}

// Block-cooperative: the residual chunk masses of row n into m[0..NC),
// recomputing missing ones and ones published as NaN.
template <bool VEC>
__device__ void gather_resid_l(const Args& a, int b, int n, const LRow& r, double* m)
{
    __shared__ unsigned long long s_miss[2];
    const int NC = a.NC, K = a.K, V = a.V;
    const unsigned ep = a.epoch;
    const unsigned long long* wp = a.wpart + ((int64_t)b * K + n) * NC;
    const int c = threadIdx.x;
    bool need = c < NC, redo = false;
    const unsigned long long t0 = wall_clock64();
    for (;;) {
        bool any = false;
        if (need) {
            const unsigned long long wv = get_u64(&wp[c]);
            if (f64_ok(wv, ep) && !a.force_recompute) {
                m[c] = f64_of(wv);
                need = false;
                if (m[c] != m[c]) redo = true;
            } else {
                any = true;
            }
        }
        if (!__syncthreads_or(any)) break;
        if (wait_expired(a, t0)) break;
        __builtin_amdgcn_s_sleep(2);
    }
    if (!__syncthreads_or(need || redo)) return;
    if (threadIdx.x < 2) s_miss[threadIdx.x] = 0ull;
    __syncthreads();
    if (need || redo) atomicOr(&s_miss[c >> 6], 1ull << (c & 63));   // LDS
    __syncthreads();
    const Row prow = row_of(a.tp + ((int64_t)b * (K + 1) + n) * V, V);
    const Row qrow = row_of(a.dp + ((int64_t)b * K + n) * V, V);
    for (int h = 0; h < 2; ++h) {
        unsigned long long mk = s_miss[h];
        while (mk) {
            const int cc = h * 64 + __ffsll((unsigned long long)mk) - 1;
            mk &= mk - 1;
            const double w = block_sum(thread_resid_reload_l<VEC>(prow, qrow, cc, V, r, a.ktau));
            if (threadIdx.x == 0) {
                m[cc] = strip8(w);
                put_u32(&a.hdr->slow_path, 1u);
            }
        }
    }
    __syncthreads();
}

// Block-cooperative: the maxima and masses of row i of sequence b (with Q,
// also its draft row), and its chunks' masses scaled to the row maximum in
// ms[0..NC) (target).  Words that do not carry this call's tag within the
// wait bound are recomputed from the inputs, bit-identically.
template <bool VEC, bool Q>
__device__ LRow gather_row_l(const Args& a, int b, int i, double* ms)
{
    __shared__ float s_mp[kMaxNC], s_mq[kMaxNC];
    __shared__ double s_sp[kMaxNC], s_sq[kMaxNC];
    __shared__ unsigned long long s_miss[2];
    __shared__ LRow s_row;
    const int NC = a.NC, K = a.K, V = a.V, c = threadIdx.x;
    const unsigned ep = a.epoch;
    const int64_t row = (int64_t)b * (K + 1) + i;
    bool need = c < NC;
    const unsigned long long t0 = wall_clock64();
    for (;;) {
        bool any = false;
        if (need) {
            const Part* pp = a.parts + row * NC + c;
            const unsigned long long sp = get_u64(&pp->sp), mp = get_u64(&pp->am);
            const unsigned long long sq = Q ? get_u64(&pp->sq) : 0ull, mq = Q ? get_u64(&pp->smin) : 0ull;
            const bool ok = f64_ok(sp, ep) && am_ok(mp, ep) && (!Q || (f64_ok(sq, ep) && am_ok(mq, ep)));
            if (ok && !a.force_recompute) {
                s_sp[c] = f64_of(sp);
                s_mp[c] = am_val(mp);
                if (Q) {
                    s_sq[c] = f64_of(sq);
                    s_mq[c] = am_val(mq);
                }
                need = false;
            } else {
                any = true;
            }
        }
        if (!__syncthreads_or(any)) break;
        if (wait_expired(a, t0)) break;
        __builtin_amdgcn_s_sleep(2);
    }
    if (__syncthreads_or(need)) {   // recompute what is missing (rare), one chunk at a time
        if (threadIdx.x < 2) s_miss[threadIdx.x] = 0ull;
        __syncthreads();
        if (need) atomicOr(&s_miss[c >> 6], 1ull << (c & 63));   // LDS
        __syncthreads();
        const Row prow = row_of(a.tp + row * V, V);
        const Row qrow = Q ? row_of(a.dp + ((int64_t)b * K + i) * V, V) : prow;
        int slot = 0;
        for (int h = 0; h < 2; ++h) {
            unsigned long long mk = s_miss[h];
            while (mk) {
                const int cc = h * 64 + __ffsll((unsigned long long)mk) - 1;
                mk &= mk - 1;
                float4 pv[kVecS], qv[kVecS];
#pragma unroll
                for (int j = 0; j < kVecS; ++j) {
                    pv[j] = load_one<VEC, kVecS>(prow, cc, j);
                    qv[j] = Q ? load_one<VEC, kVecS>(qrow, cc, j) : pv[j];
                }
                const LStat st = chunk_stats_l<kVecS, Q>(pv, qv, cc, V, a.ktau, slot);
                slot ^= 1;
                if (threadIdx.x == 0) {
                    s_sp[cc] = strip8(st.sp);
                    s_mp[cc] = st.mp;
                    if (Q) {
                        s_sq[cc] = strip8(st.sq);
                        s_mq[cc] = st.mq;
                    }
                    put_u32(&a.hdr->slow_path, 1u);
                }
            }
        }
        __syncthreads();
    }
    if (threadIdx.x < 64) {
        const int l = threadIdx.x;
        const float m0 = l < NC ? s_mp[l] : -INFINITY, m1 = l + 64 < NC ? s_mp[l + 64] : -INFINITY;
        const double x0 = l < NC ? s_sp[l] : 0.0, x1 = l + 64 < NC ? s_sp[l + 64] : 0.0;
        LRow r{0.0, 0.0, 0.0f, 0.0f};
        r.P = row_mass_l(m0, x0, m1, x1, a.ktau, &r.Mp);
        if (l < NC) ms[l] = chunk_scaled(m0, x0, r.Mp, a.ktau);
        if (l + 64 < NC) ms[l + 64] = chunk_scaled(m1, x1, r.Mp, a.ktau);
        if (Q) {
            const float n0 = l < NC ? s_mq[l] : -INFINITY, n1 = l + 64 < NC ? s_mq[l + 64] : -INFINITY;
            const double y0 = l < NC ? s_sq[l] : 0.0, y1 = l + 64 < NC ? s_sq[l + 64] : 0.0;
            r.Q = row_mass_l(n0, y0, n1, y1, a.ktau, &r.Mq);
        }
        if (l == 0) s_row = r;
    }
    __syncthreads();
    return s_row;
}

// Search of chunk c (the chunk_draw search) with logit weights: the residual
// max(0, w_p Q - w_q P) (RESID) or w_p, against the row maxima; positions at
// or past V weigh 0.
template <bool VEC, bool RESID>
__device__ __forceinline__ int chunk_draw_l(Row prow, Row qrow, const LRow& r, float k, int V, int c, double base,
                                            double T)
{
    constexpr int NV = kVecS;
    __shared__ double s_seg[NV][kWaves];
    __shared__ int s_ks, s_ws;
    __shared__ double s_base;
    __shared__ int s_x;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    auto wt = [&](float p, float q, int pos) -> double {
        if (pos >= V) return 0.0;
        return RESID ? resid_l(p, q, r.P, r.Q, r.Mp, r.Mq, k) : (double)lweight(p, r.Mp, k);
    };
    float4 pv[NV], qv[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        pv[j] = load_one<VEC, NV>(prow, c, j);
        qv[j] = RESID ? load_one<VEC, NV>(qrow, c, j) : pv[j];
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int p0 = 4 * f4_index<NV>(c, j);
        double t = 0.0;
#pragma unroll
        for (int e = 0; e < 4; ++e) t += wt(comp(pv[j], e), comp(qv[j], e), p0 + e);
        const double s = wave_sum(t);
        if (lane == 0) s_seg[j][w] = s;
    }
    __syncthreads();
    if (threadIdx.x < 64) {
        constexpr int kSegs = NV * kWaves;
        const int q = threadIdx.x;
        const double s = q < kSegs ? s_seg[q / kWaves][q % kWaves] : 0.0;
        const double incl = wave_inclusive_scan(s);
        double excl = __shfl_up(incl, 1);
        if (q == 0) excl = 0.0;
        const double run = base + excl;
        const unsigned long long mh = __ballot(q < kSegs && run + s > T);
        const unsigned long long mp = __ballot(q < kSegs && s > 0.0);
        const int sel = mh ? __ffsll((unsigned long long)mh) - 1 : (mp ? 63 - __clzll(mp) : 0);
        const double bs = __shfl(run, sel);
        if (q == 0) {
            s_ks = sel / kWaves;
            s_ws = sel % kWaves;
            s_base = bs;
        }
    }
    __syncthreads();
    if (w == s_ws) {
        const int j = s_ks;
        float4 p4 = pv[0], q4 = qv[0];
#pragma unroll
        for (int jj = 1; jj < NV; ++jj)
            if (jj == j) {
                p4 = pv[jj];
                q4 = qv[jj];
            }
        const int p0 = 4 * f4_index<NV>(c, j);
        double vv[4], tot = 0.0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            vv[e] = wt(comp(p4, e), comp(q4, e), p0 + e);
            tot += vv[e];
        }
        const double incl = wave_inclusive_scan(tot);
        double run = __shfl_up(incl, 1);
        if (lane == 0) run = 0.0;
        run += s_base;
        int hit = -1, lastpos = -1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            run += vv[e];
            if (hit < 0 && run > T) hit = e;
            if (vv[e] > 0.0) lastpos = e;
        }
        const unsigned long long mh = __ballot(hit >= 0);
        if (mh) {
            const int l = __ffsll((unsigned long long)mh) - 1;
            if (lane == l) s_x = p0 + hit;
        } else {
            const unsigned long long mp = __ballot(lastpos >= 0);
            if (mp) {
                const int l = 63 - __clzll(mp);
                if (lane == l) s_x = p0 + lastpos;
            } else if (lane == 0) {
                s_x = p0;   // unreachable for a segment with mass
            }
        }
    }
    __syncthreads();
    return s_x;
}

// Block-cooperative: the final draw of sequence b once n and row n's masses
// are known (r: row n; for n == K only its target part is read), and the
// outputs.  n < K: the residual of row n, located by the published residual
// chunk masses; n == K (or a rejection that left no residual mass): the
// warped target row n, located by its scaled chunk masses.
template <bool VEC>
__device__ void draw_and_write_l(const Args& a, int b, int n, LRow r)
{
    __shared__ double s_m[kMaxNC];
    __shared__ int s_owner, s_resid;
    __shared__ double s_base, s_T;
    const int NC = a.NC, K = a.K, V = a.V;
    const int64_t row0 = (int64_t)b * (K + 1);
    const double uK = (double)a.u[row0 + K];
    const Row prow = row_of(a.tp + (row0 + n) * V, V);
    const Row qrow = n < K ? row_of(a.dp + ((int64_t)b * K + n) * V, V) : prow;
    if (n < K) gather_resid_l<VEC>(a, b, n, r, s_m);
    if (threadIdx.x < 64) {
        int owner = -1;
        double base = 0.0, T = 0.0, W = 0.0;
        if (n < K) W = locate_chunk(s_m, NC, uK, &owner, &base, &T);
        if (threadIdx.x == 0) {
            s_owner = owner;
            s_base = base;
            s_T = T;
            s_resid = (n < K && W > 0.0) ? 1 : 0;
        }
    }
    __syncthreads();
    const int resid_draw = s_resid;
    if (!resid_draw) {
        const LRow rp = gather_row_l<VEC, false>(a, b, n, s_m);
        r.Mp = rp.Mp;
        if (threadIdx.x < 64) {
            int owner;
            double base, T;
            locate_chunk(s_m, NC, uK, &owner, &base, &T);
            if (threadIdx.x == 0) {
                s_owner = owner;
                s_base = base;
                s_T = T;
            }
        }
        __syncthreads();
    }
    int x = -1;
    if (s_owner >= 0)
        x = resid_draw ? chunk_draw_l<VEC, true>(prow, qrow, r, a.ktau, V, s_owner, s_base, s_T)
                       : chunk_draw_l<VEC, false>(prow, prow, r, a.ktau, V, s_owner, s_base, s_T);
    if (threadIdx.x == 0) {
        a.n_out[b] = n;
        a.next_out[b] = x;
    }
    __syncthreads();
}

// The decision of sequence b taken by its finishing block when the walks
// could not take it: the accept-prefix length n and the masses of row n.
struct LDecision {
    LRow r;
    int n;
};

// Block-cooperative, for a sequence whose walks could not decide (rare):
// the decisions from the gathered (or recomputed) partials, row by row.  Not
// inlined, so that this rarely taken code stays out of the register
// allocation of the walks.
template <bool VEC>
__device__ __noinline__ LDecision decide_rows_l(const Args& a, int b)
{
    __shared__ double s_unused[kMaxNC];
    __shared__ int s_rej;
    const int K = a.K, V = a.V;
    const int64_t row0 = (int64_t)b * (K + 1);
    LDecision d{LRow{0.0, 0.0, 0.0f, 0.0f}, K};
    for (int i = 0; i < K; ++i) {
        const LRow r = gather_row_l<VEC, true>(a, b, i, s_unused);
        if (threadIdx.x == 0) {
            const int tk = a.dt[(int64_t)b * K + i];
            const bool tin = tk >= 0 && tk < V;
            s_rej = accepted_l(tin, a.u[row0 + i], tin ? a.tp[(row0 + i) * V + tk] : 0.0f,
                               tin ? a.dp[((int64_t)b * K + i) * V + tk] : 0.0f, r, a.ktau, a.ktau64) ? 0 : 1;
        }
        __syncthreads();
        const int rej = s_rej;
        __syncthreads();
        if (rej) {
            d.n = i;
            d.r = r;
            break;
        }
    }
    return d;
}

// Block-cooperative: the outcome the walks of sequence b published (n + 1,
// or 0 when they could not decide), or 0 when it does not arrive within the
// wait bound.
__device__ int wait_state_l(const Args& a, int b)
{
    __shared__ int s_code;
    const unsigned long long t0 = wall_clock64();
    for (;;) {
        bool got = false;
        if (threadIdx.x == 0) {
            const unsigned long long v = get_u64(&a.sstate[b]);
            got = f64_ok(v, a.epoch) && !a.force_recompute;
            const unsigned long long code = v >> 8;
            s_code = got && code <= (unsigned long long)(a.K + 1) ? (int)code : 0;   // 0: decide here
        }
        if (__syncthreads_or(got)) break;
        if (wait_expired(a, t0)) break;
        __builtin_amdgcn_s_sleep(2);
    }
    const int code = s_code;
    __syncthreads();
    return code;
}

template <bool VEC, bool ROWS, bool EARLY = false>
__global__ __launch_bounds__(kThreads, 4) void sv_logits_kernel(Args a)
{
    const int NC = a.NC, K = a.K, V = a.V;
    const float kt = a.ktau;
    // The finishing block of a sequence draws from row dn (with masses dr)
    // at the end: one draw serves the walk that found a rejection and the
    // bonus block that finishes a fully accepted (or undecided) sequence.
    int b, dn = -1;
    LRow dr{0.0, 0.0, 0.0f, 0.0f};
    int walk_code = -1;   // set by a finishing walk: n + 1, or 0 if it could not decide

    if (blockIdx.x >= a.nwalk) {
        // bonus row K (target only), two chunks per block
        const int per_seq = (NC + kBonusChunks - 1) / kBonusChunks;
        const unsigned blk = blockIdx.x - a.nwalk;
        b = (int)(blk / (unsigned)per_seq);
        const int c0 = (int)(blk - (unsigned)b * (unsigned)per_seq) * kBonusChunks;
        const int64_t row0 = (int64_t)b * (K + 1);
        if (EARLY && K > 0) {
            // early exit: skip the bonus row once the walks' outcome shows a
            // rejection (as in sv_sample_kernel)
            __shared__ int s_skip;
            if (threadIdx.x == 0) {
                const unsigned long long v = get_u64(&a.sstate[b]);
                const unsigned long long code = v >> 8;
                s_skip = f64_ok(v, a.epoch) && !a.force_recompute && code >= 1 && code <= (unsigned long long)K;
            }
            __syncthreads();
            if (s_skip) return;
        }
        const Row prow = row_of(a.tp + (row0 + K) * V, V);
        float4 xp[kBonusChunks][kVecS];
#pragma unroll
        for (int j = 0; j < kBonusChunks; ++j)   // chunks past NC read as zeros and are masked
            load_chunk_keep<VEC, kVecS>(prow, c0 + j < NC ? c0 + j : NC, xp[j],
                                        blk + kTailBlocks >= gridDim.x - a.nwalk);
#pragma unroll
        for (int j = 0; j < kBonusChunks; ++j) {
            const int cj = c0 + j < NC ? c0 + j : NC;
            const LStat st = chunk_stats_l<kVecS, false>(xp[j], xp[j], cj, V, kt, j & 1);
            if (c0 + j < NC) publish_l(a, row0 + K, c0 + j, st, false);
        }
        const int fc = finisher_column(b, NC);
        if (fc < c0 || fc >= c0 + kBonusChunks) return;
        // the block of the finishing column finishes the sequence once the
        // walks' outcome is there: after full acceptance (or K == 0) it draws
        // the bonus token; after a rejection the finishing walk has drawn.
        // Row blocks publish no outcome: this block then decides itself.
        __builtin_amdgcn_s_setprio(3);
        const int code = K == 0 ? K + 1 : ROWS ? 0 : wait_state_l(a, b);
        if (code == K + 1) {
            dn = K;
        } else if (code <= 0) {
            // the callee reads the arguments where the kernel received
            // them, so the kernel keeps no copy of them in scratch memory
            const Args& ka = *(const Args*)(const void*)__builtin_amdgcn_kernarg_segment_ptr();
            const LDecision d = decide_rows_l<VEC>(ka, b);
            dn = d.n;
            dr = d.r;
        } else {
            return;
        }
    } else if (ROWS) {
        // one block per (sequence b, draft row i, chunk c), as in the row
        // form of sv_sample_kernel
        const unsigned w = blockIdx.x / (unsigned)NC;
        b = (int)(w / (unsigned)K);
        const int i = (int)(w - (unsigned)b * (unsigned)K);
        const int c = (int)(blockIdx.x - w * (unsigned)NC);
        const int64_t row = (int64_t)b * (K + 1) + i;
        float4 xp[kVecS], xq[kVecS];
        load_chunk<VEC, kVecS>(row_of(a.tp + row * V, V), c, xp);
        load_chunk<VEC, kVecS>(row_of(a.dp + ((int64_t)b * K + i) * V, V), c, xq);
        const int tok = threadIdx.x == 0 ? a.dt[(int64_t)b * K + i] : -1;
        publish_l(a, row, c, chunk_stats_l<kVecS, true>(xp, xq, c, V, kt, 0), true);
        park(xp, xq);
        LRow r;
        PollL pl = poll_issue_l(a, b, i, tok);
        settle_poll_l(pl);
        const int rej = poll_decide_l(a, b, i, pl, &r);
        if (rej != 0) {   // rejected: the residual mass; undecided: marked for recomputing
            const double m = rej > 0 ? block_sum(parked_resid_l(r, kt, c, V)) : __builtin_nan("");
            if (threadIdx.x == 0) put_u64(&a.wpart[((int64_t)b * K + i) * NC + c], tag_f64(m, a.epoch));
        }
        return;
    } else {
    // a walk: chunk column c of draft rows 0..K-1 of sequence b (K >= 1)
    b = (int)(blockIdx.x / (unsigned)NC);
    const int c = (int)(blockIdx.x - (unsigned)b * (unsigned)NC);
    const float* tb = a.tp + (int64_t)b * (K + 1) * V;
    const float* db = a.dp + (int64_t)b * K * V;
    const int64_t row0 = (int64_t)b * (K + 1);
    int state = kSearching;
    LRow rn{0.0, 0.0, 0.0f, 0.0f};
    int tok = -1;
    float4 xp[kVecS], xq[kVecS], yp[kVecS], yq[kVecS];
    __builtin_amdgcn_s_setprio(2);   // searching walks first, as in the probabilities walk (236.3 -> 235.0 us)
    load_chunk<VEC, kVecS>(row_of(tb, V), c, xp);
    load_chunk<VEC, kVecS>(row_of(db, V), c, xq);

    auto decide = [&](int j, const PollL& pl) {
        LRow r;
        const int rej = poll_decide_l(a, b, j, pl, &r);
        if (rej < 0) {
            state = kLost;
            if (threadIdx.x == 0)
                for (int q = j; q < K; ++q)
                    put_u64(&a.wpart[((int64_t)b * K + q) * NC + c], tag_f64(__builtin_nan(""), a.epoch));
        } else if (rej) {
            state = j;
            rn = r;
            const double w = block_sum(parked_resid_l(r, kt, c, V));
            if (threadIdx.x == 0) put_u64(&a.wpart[((int64_t)b * K + j) * NC + c], tag_f64(w, a.epoch));
        }
    };
    // Row i+1's loads into (p, q) (an empty range after the last draft row
    // reads zeros).  The logits walk keeps its two row buffers by turns: the
    // row of one step is computed where the previous step loaded it, so the
    // next row's loads leave without first waiting for that row and copying
    // it over (the arithmetic of a logits row is long enough for this to
    // show: 232.2 -> 229.6 us at B=256 K=5 V=128256; the probabilities walk
    // measured no difference).  Functions taking the buffers are inlined:
    // out of line they would take the kernel arguments' address.
    auto load_to = [&](int i, float4 (&p)[kVecS], float4 (&q)[kVecS]) __attribute__((always_inline)) {
        const bool more = i + 1 < K;
        const int64_t off = more ? (int64_t)(i + 1) * V : 0;
        load_chunk<VEC, kVecS>(row_of(tb + off, more ? V : 0), c, p);
        load_chunk<VEC, kVecS>(row_of(db + off, more ? V : 0), c, q);
    };
    // one searching step: row i in (cp, cq), row i+1 loading into (np, nq)
    auto search_step = [&](int i, float4 (&cp)[kVecS], float4 (&cq)[kVecS], float4 (&np)[kVecS],
                           float4 (&nq)[kVecS]) __attribute__((always_inline)) {
        PollL pl{0ull, 0ull, 0ull, 0ull, 0.0f, 0.0f, 0.0f, 0};
        const bool pending = i > 0;
        if (pending) pl = poll_issue_l(a, b, i - 1, tok);
        if (threadIdx.x == 0) tok = a.dt[(int64_t)b * K + i];
        __builtin_amdgcn_sched_barrier(0);
        if (!EARLY) load_to(i, np, nq);
        __builtin_amdgcn_sched_barrier(0);
        publish_l(a, row0 + i, c, chunk_stats_l<kVecS, true>(cp, cq, c, V, kt, i & 1), true);
        if (pending) {
            settle_poll_l(pl);
            decide(i - 1, pl);
        }
        if (EARLY && state < 0) load_to(i, np, nq);   // early exit: loads after the decision (searching or lost)
        if (state == kSearching) park(cp, cq);
    };

    int i = 0;
    while (i < K) {   // two steps a turn; the row of the step after the loop is left in (xp, xq)
        search_step(i, xp, xq, yp, yq);
        ++i;
        if (state != kSearching || i >= K) {
#pragma unroll
            for (int j = 0; j < kVecS; ++j) {
                xp[j] = yp[j];
                xq[j] = yq[j];
            }
            break;
        }
        search_step(i, yp, yq, xp, xq);
        ++i;
        if (state != kSearching) break;
    }
    if (EARLY && state >= 0) i = K;   // early exit: no row after a decided rejection
    __builtin_amdgcn_s_setprio(0);
    for (; i + 1 < K; i += 2) {   // streaming, also two rows a turn
        load_to(i, yp, yq);
        __builtin_amdgcn_sched_barrier(0);
        publish_l(a, row0 + i, c, chunk_stats_l<kVecS, true>(xp, xq, c, V, kt, i & 1), true);
        load_to(i + 1, xp, xq);
        __builtin_amdgcn_sched_barrier(0);
        publish_l(a, row0 + i + 1, c, chunk_stats_l<kVecS, true>(yp, yq, c, V, kt, (i + 1) & 1), true);
    }
    if (i < K) {
        load_to(i, yp, yq);
        __builtin_amdgcn_sched_barrier(0);
        publish_l(a, row0 + i, c, chunk_stats_l<kVecS, true>(xp, xq, c, V, kt, i & 1), true);
        ++i;
    }
    if (state == kSearching) {
        PollL pl = poll_issue_l(a, b, K - 1, tok);
        settle_poll_l(pl);
        decide(K - 1, pl);
        if (state == kSearching) state = K;
    }
    if (c != finisher_column(b, NC)) return;
    __builtin_amdgcn_s_setprio(3);
    walk_code = state >= 0 ? state + 1 : 0;
    if (state >= 0 && state < K) {
        dn = state;
        dr = rn;
    }
    }
    if (dn >= 0) draw_and_write_l<VEC>(a, b, dn, dr);
    // the walks' outcome, for the bonus block that finishes the sequence:
    // n + 1 (the draw is then made when n < K), 0 when they could not decide
    if (walk_code >= 0 && threadIdx.x == 0) put_u64(&a.sstate[b], tag_state(walk_code, a.epoch));
}

__global__ void sv_fill_zero_kernel(uint4* p, size_t n16)
{
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    for (size_t j = (size_t)blockIdx.x * blockDim.x + threadIdx.x; j < n16; j += (size_t)gridDim.x * blockDim.x)
        p[j] = z;
}

// ------------------------------------------------------------- host --

struct DevInfo {
    int wall_khz = 0;
    bool ok = false;
};

std::mutex g_mu;
DevInfo g_dev[64];
struct WsState {
    unsigned calls = 0;      // calls since the last clear (tags 1..calls are in use)
    size_t bytes = 0;        // largest extent of the workspace seen
};
std::unordered_map<const void*, WsState> g_ws;

struct Tuning {
    double poll_us = kPollMicroseconds;
    int force_recompute = 0;
    int rows = -1;           // sampled form: -1 by size, 0 walks, 1 one block per row
    int force_lost = 0;
};

// Read at every call: SV_VERIFY_POLL_US bounds a wait for a sibling's
// partials; SV_VERIFY_FORCE_RECOMPUTE=1 makes every reader recompute what it
// gathers (a test hook for the recompute path); SV_VERIFY_FORCE_LOST=1 makes
// every decision taken inside a walk or row block report that its partials
// did not arrive, while the readers that finish a sequence still trust the
// published words (a test hook for the lost-decision path).
Tuning tuning()
{
    Tuning r;
    if (const char* s = std::getenv("SV_VERIFY_POLL_US")) r.poll_us = std::atof(s);
    if (const char* s = std::getenv("SV_VERIFY_FORCE_RECOMPUTE")) r.force_recompute = std::atoi(s) != 0;
    if (const char* s = std::getenv("SV_VERIFY_ROWS")) r.rows = std::atoi(s) != 0 ? 1 : 0;
    if (const char* s = std::getenv("SV_VERIFY_FORCE_LOST")) r.force_lost = std::atoi(s) != 0;
    if (!(r.poll_us >= 0.0) || r.poll_us > 1e7) r.poll_us = kPollMicroseconds;
    return r;
}

sv_status device_info(DevInfo* out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return SV_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    DevInfo& d = g_dev[dev];
    if (!d.ok) {
        int khz = 0;
        if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
            khz = 100000;   // gfx9 wall clock: 100 MHz
        d.wall_khz = khz;
        d.ok = true;
    }
    *out = d;
    return SV_OK;
}

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// The form of a sampled pass: one block per draft row for small grids, walks
// down the rows otherwise.  A walk's latency grows with its K rows, the row
// form's with the waves of blocks it takes to fill the chip (its blocks wait
// for their row's siblings), so the limit grows with K: up to
// per_draft_row * max(4, K) blocks, where the row form measured faster or
// equal (512 on probabilities; 256 on logits, where every rejected row, not
// only the first, pays a residual of two exp2 per value).  Both forms take
// the same decisions from the same words: the outputs do not depend on the
// form.  SV_VERIFY_ROWS forces one (a test hook).
bool use_rows(int K, uint64_t per_row, uint64_t bonus, uint64_t per_draft_row, const Tuning& tu)
{
    if (K <= 0) return false;
    if (tu.rows >= 0) return tu.rows == 1;
    return (uint64_t)K * per_row + bonus <= per_draft_row * (uint64_t)(K > 4 ? K : 4);
}

// The greedy kernel needs little LDS, so up to 8 of its blocks would share a
// CU; measured, 4 (the residency of the sampled pass) streams faster: 8192-
// value chunks at B=256 K=5 V=128256 take 115 instead of 118 µs, at B=32 K=16
// V=262144 83.4 instead of 85.1 µs (3 per CU: 123 and 89 µs).  A launch of
// more blocks than fit at once uncapped (8 per CU) therefore asks for dynamic
// LDS up to kGreedyLdsPerBlock per block: 4 x 36 KB fit in a CU's 160 KB, 5
// do not.  A smaller grid (B=64 K=4 V=32000: 1280 blocks) stays uncapped, all
// of it resident at once.  The kernel's own static LDS is read once.
template <bool VEC, bool STATS>
unsigned greedy_lds_pad()
{
    static const unsigned pad = [] {
        hipFuncAttributes fa{};
        if (hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(&sv_greedy_kernel<VEC, STATS>)) != hipSuccess) {
            (void)hipGetLastError();   // no pad then; the launch must not report this query's error
            return 0u;
        }
        return fa.sharedSizeBytes < kGreedyLdsPerBlock ? (unsigned)(kGreedyLdsPerBlock - fa.sharedSizeBytes) : 0u;
    }();
    return pad;
}

template <bool VEC, bool STATS>
void launch_greedy(dim3 grid, hipStream_t s, const Args& a)
{
    const unsigned pad = grid.x > kGreedyUncappedBlocks ? greedy_lds_pad<VEC, STATS>() : 0u;
    hipLaunchKernelGGL((sv_greedy_kernel<VEC, STATS>), grid, dim3(kThreads), pad, s, a);
}

template <bool VEC, bool STATS>
void launch_sample(bool rows, dim3 grid, hipStream_t s, const Args& a)
{
    if (rows)
        hipLaunchKernelGGL((sv_sample_kernel<VEC, STATS, true>), grid, dim3(kThreads), 0, s, a);
    else if (!STATS && a.early)
        hipLaunchKernelGGL((sv_sample_kernel<VEC, false, false, true>), grid, dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((sv_sample_kernel<VEC, STATS, false>), grid, dim3(kThreads), 0, s, a);
}

sv_status check_sizes(int32_t B, int32_t K, int32_t V)
{
    if (B < 0 || K < 0 || V < 1) return SV_ERR_INVALID_ARG;
    if (V > SV_MAX_V || K > SV_MAX_K) return SV_ERR_UNSUPPORTED;
    const uint64_t NC = ((uint64_t)V + kChunkS - 1) / kChunkS;   // the larger chunk count
    if ((uint64_t)B * (uint64_t)(K + 1) * NC >= (1ull << 31)) return SV_ERR_UNSUPPORTED;
    return SV_OK;
}

sv_status launch_fill(void* ws, size_t bytes, hipStream_t s)
{
    const size_t n16 = bytes / 16;
    if (n16 == 0) return SV_OK;
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(sv_fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<uint4*>(ws), n16);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

// The tag of this call on `ws` (1..kEpochs).  Each tag is used once between
// clears: the first call on a workspace the library has not seen, a call
// with more bytes than any earlier call at that address (the new part was
// never cleared), and every call after kEpochs tags have been used clear the
// whole extent of the workspace seen so far on `s` first, so no word left by
// an earlier call can carry a tag in use.  `fixed` (the static scratch)
// holds its own state, so that call takes no map entry.
sv_status next_epoch(void* ws, size_t bytes, hipStream_t s, unsigned* ep, WsState* fixed = nullptr)
{
    bool clear = false;
    size_t extent = 0;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        WsState* stp = fixed;
        if (!stp) {
            auto it = g_ws.find(ws);
            if (it == g_ws.end()) {
                it = g_ws.emplace(ws, WsState{}).first;
                it->second.calls = kEpochs;   // unknown contents: clear first
            }
            stp = &it->second;
        }
        WsState& st = *stp;
        if (bytes > st.bytes) {   // the part beyond the extent cleared so far holds unknown words
            st.bytes = bytes;
            st.calls = kEpochs;
        }
        if (st.calls >= kEpochs) {
            st.calls = 0;
            clear = true;
        }
        *ep = ++st.calls;
        extent = st.bytes;
    }
    return clear ? launch_fill(ws, extent, s) : SV_OK;
}

// Per device: the device address of `scratch` and the tag state of that
// array, filled by the first no-allocation call on the device.
struct ScratchDev {
    void* ptr = nullptr;
    WsState st;
};
ScratchDev g_scratch[64];

// The current device's copy of `scratch` (looked up once per device, with
// that device current) and its tag state.
sv_status scratch_of_device(void** ptr, WsState** state)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return SV_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    ScratchDev& d = g_scratch[dev];
    if (!d.ptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return SV_ERR_HIP;
        }
        d.ptr = p;
        d.st.calls = kEpochs;   // contents unknown: the first call clears what it uses
        d.st.bytes = 0;
    }
    *ptr = d.ptr;
    *state = &d.st;
    return SV_OK;
}

Args make_args(void* ws, int32_t B, int32_t K, int32_t V, bool sampled)
{
    Args a{};
    const int NC = (V + chunk_of(sampled) - 1) / chunk_of(sampled);
    const Layout L = make_layout(B, K, NC, sampled);
    unsigned char* w = static_cast<unsigned char*>(ws);
    a.hdr = reinterpret_cast<Header*>(w + L.hdr);
    a.parts = reinterpret_cast<Part*>(w + L.parts);
    a.wpart = reinterpret_cast<unsigned long long*>(w + L.wpart);
    a.sstate = reinterpret_cast<unsigned long long*>(w + L.sstate);
    a.B = B;
    a.K = K;
    a.V = V;
    a.NC = NC;
    return a;
}

}  // namespace

namespace {
sv_status check_sample_args(const float* target_probs, const float* draft_probs,
                            const int32_t* draft_tokens, const float* uniforms,
                            int32_t B, int32_t K, int32_t V,
                            const int32_t* n_accepted, const int32_t* next_token, const sv_row_stats* stats);
// The body of both sampled entry points (early: the early-exit form).
sv_status sample_call(const float* target_probs, const float* draft_probs,
                      const int32_t* draft_tokens, const float* uniforms,
                      int32_t B, int32_t K, int32_t V,
                      int32_t* n_accepted, int32_t* next_token,
                      void* workspace, size_t workspace_bytes,
                      sv_row_stats* stats, void* stream, bool early, WsState* fixed = nullptr);
// The body of both logits entry points.
sv_status logits_call(const float* target_logits, const float* draft_logits,
                      const int32_t* draft_tokens, const float* uniforms, float temperature,
                      int32_t B, int32_t K, int32_t V,
                      int32_t* n_accepted, int32_t* next_token,
                      void* workspace, size_t workspace_bytes, void* stream, bool early);
}   // namespace

extern "C" {

size_t sv_workspace_size(int32_t B, int32_t K, int32_t V, int32_t sampled)
{
    if (check_sizes(B, K, V) != SV_OK) return 0;
    const bool s = sampled != 0;
    const int NC = (V + chunk_of(s) - 1) / chunk_of(s);
    return make_layout(B, K, NC, s).total;
}

sv_status sv_workspace_init(void* workspace, size_t workspace_bytes, void* stream)
{
    if (!workspace || !aligned(workspace, 16)) return SV_ERR_WORKSPACE;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        WsState& st = g_ws[workspace];
        st.calls = 0;
        st.bytes = workspace_bytes;
    }
    return launch_fill(workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

sv_status sv_verify_greedy_batched(const float* target_probs, const int32_t* draft_tokens,
                                   int32_t B, int32_t K, int32_t V,
                                   int32_t* n_accepted, int32_t* next_token,
                                   void* workspace, size_t workspace_bytes,
                                   sv_row_stats* stats, void* stream)
{
    sv_status st = check_sizes(B, K, V);
    if (st != SV_OK) return st;
    if (B == 0) return SV_OK;   // nothing to verify; pointers are not inspected
    if (!target_probs || !n_accepted || !next_token || (K > 0 && !draft_tokens))
        return SV_ERR_INVALID_ARG;
    if (!aligned(target_probs, 4) || !aligned(draft_tokens, 4) || !aligned(n_accepted, 4) ||
        !aligned(next_token, 4) || !aligned(stats, 8))
        return SV_ERR_INVALID_ARG;
    if (!workspace || !aligned(workspace, 16) || workspace_bytes < sv_workspace_size(B, K, V, 0))
        return SV_ERR_WORKSPACE;
    DevInfo d;
    st = device_info(&d);
    if (st != SV_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Args a = make_args(workspace, B, K, V, false);
    st = next_epoch(workspace, workspace_bytes, s, &a.epoch);
    if (st != SV_OK) return st;
    a.tp = target_probs;
    a.dt = draft_tokens;
    a.n_out = n_accepted;
    a.next_out = next_token;
    a.stats = stats;
    const Tuning tu = tuning();
    a.force_recompute = tu.force_recompute;
    a.force_lost = tu.force_lost;
    a.poll_ticks = (unsigned long long)(tu.poll_us * 1e-3 * (double)d.wall_khz);
    const bool vec = (V % 4 == 0) && aligned(target_probs, 16);
    const dim3 grid((unsigned)((uint64_t)B * (uint64_t)(K + 1) * (uint64_t)a.NC));
    if (vec && stats)
        launch_greedy<true, true>(grid, s, a);
    else if (vec)
        launch_greedy<true, false>(grid, s, a);
    else if (stats)
        launch_greedy<false, true>(grid, s, a);
    else
        launch_greedy<false, false>(grid, s, a);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status sv_verify_sample_batched(const float* target_probs, const float* draft_probs,
                                   const int32_t* draft_tokens, const float* uniforms,
                                   int32_t B, int32_t K, int32_t V,
                                   int32_t* n_accepted, int32_t* next_token,
                                   void* workspace, size_t workspace_bytes,
                                   sv_row_stats* stats, void* stream)
{
    return sample_call(target_probs, draft_probs, draft_tokens, uniforms, B, K, V, n_accepted, next_token,
                       workspace, workspace_bytes, stats, stream, false);
}

sv_status sv_verify_sample_early_batched(const float* target_probs, const float* draft_probs,
                                         const int32_t* draft_tokens, const float* uniforms,
                                         int32_t B, int32_t K, int32_t V,
                                         int32_t* n_accepted, int32_t* next_token,
                                         void* workspace, size_t workspace_bytes, void* stream)
{
    return sample_call(target_probs, draft_probs, draft_tokens, uniforms, B, K, V, n_accepted, next_token,
                       workspace, workspace_bytes, nullptr, stream, true);
}

sv_status sv_verify_sample_batched_noalloc(const float* target_probs, const float* draft_probs,
                                           const int32_t* draft_tokens, const float* uniforms,
                                           int32_t B, int32_t K, int32_t V,
                                           int32_t* n_accepted, int32_t* next_token,
                                           sv_row_stats* stats, void* stream)
{
    const sv_status st = check_sample_args(target_probs, draft_probs, draft_tokens, uniforms, B, K, V,
                                           n_accepted, next_token, stats);
    if (st != SV_OK || B == 0) return st;
    const size_t need = sv_workspace_size(B, K, V, 1);
    if (need > (size_t)SV_SCRATCH_BYTES) return SV_ERR_SCRATCH;
    void* ws = nullptr;
    WsState* state = nullptr;
    const sv_status ss = scratch_of_device(&ws, &state);
    if (ss != SV_OK) return ss;
    return sample_call(target_probs, draft_probs, draft_tokens, uniforms, B, K, V, n_accepted, next_token,
                       ws, need, stats, stream, false, state);
}
}   // extern "C"

namespace {
// The argument checks of the sampled calls (sizes, NULL and misaligned
// pointers), before anything else is done.
sv_status check_sample_args(const float* target_probs, const float* draft_probs,
                            const int32_t* draft_tokens, const float* uniforms,
                            int32_t B, int32_t K, int32_t V,
                            const int32_t* n_accepted, const int32_t* next_token, const sv_row_stats* stats)
{
    const sv_status st = check_sizes(B, K, V);
    if (st != SV_OK) return st;
    if (B == 0) return SV_OK;   // nothing to verify; pointers are not inspected
    if (!target_probs || !uniforms || !n_accepted || !next_token ||
        (K > 0 && (!draft_probs || !draft_tokens)))
        return SV_ERR_INVALID_ARG;
    if (!aligned(target_probs, 4) || !aligned(draft_probs, 4) || !aligned(draft_tokens, 4) ||
        !aligned(uniforms, 4) || !aligned(n_accepted, 4) || !aligned(next_token, 4) ||
        !aligned(stats, 8))
        return SV_ERR_INVALID_ARG;
    return SV_OK;
}

sv_status sample_call(const float* target_probs, const float* draft_probs,
                      const int32_t* draft_tokens, const float* uniforms,
                      int32_t B, int32_t K, int32_t V,
                      int32_t* n_accepted, int32_t* next_token,
                      void* workspace, size_t workspace_bytes,
                      sv_row_stats* stats, void* stream, bool early, WsState* fixed)
{
    sv_status st = check_sample_args(target_probs, draft_probs, draft_tokens, uniforms, B, K, V, n_accepted,
                                      next_token, stats);
    if (st != SV_OK || B == 0) return st;
    if (!workspace || !aligned(workspace, 16) || workspace_bytes < sv_workspace_size(B, K, V, 1))
        return SV_ERR_WORKSPACE;
    DevInfo d;
    st = device_info(&d);
    if (st != SV_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Args a = make_args(workspace, B, K, V, true);
    st = next_epoch(workspace, workspace_bytes, s, &a.epoch, fixed);
    if (st != SV_OK) return st;
    a.tp = target_probs;
    a.dp = draft_probs;
    a.dt = draft_tokens;
    a.u = uniforms;
    a.n_out = n_accepted;
    a.next_out = next_token;
    a.stats = stats;
    a.early = early ? 1 : 0;
    const Tuning tu = tuning();
    a.force_recompute = tu.force_recompute;
    a.force_lost = tu.force_lost;
    a.poll_ticks = (unsigned long long)(tu.poll_us * 1e-3 * (double)d.wall_khz);
    const bool vec = (V % 4 == 0) && aligned(target_probs, 16) && (K == 0 || aligned(draft_probs, 16));
    const uint64_t per_row = (uint64_t)B * (uint64_t)a.NC;
    const uint64_t bonus = (uint64_t)B * (uint64_t)((a.NC + kBonusChunks - 1) / kBonusChunks);
    const bool rows = use_rows(K, per_row, bonus, kRowsBlocksPerRow, tu);
    a.nwalk = (unsigned)(K > 0 ? (rows ? (uint64_t)K * per_row : per_row) : 0);   // then the bonus-row blocks
    const dim3 grid((unsigned)(a.nwalk + bonus));
    if (vec && stats)
        launch_sample<true, true>(rows, grid, s, a);
    else if (vec)
        launch_sample<true, false>(rows, grid, s, a);
    else if (stats)
        launch_sample<false, true>(rows, grid, s, a);
    else
        launch_sample<false, false>(rows, grid, s, a);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}
}   // namespace

extern "C" {

sv_status sv_verify_sample_logits_batched(const float* target_logits, const float* draft_logits,
                                          const int32_t* draft_tokens, const float* uniforms, float temperature,
                                          int32_t B, int32_t K, int32_t V,
                                          int32_t* n_accepted, int32_t* next_token,
                                          void* workspace, size_t workspace_bytes, void* stream)
{
    return logits_call(target_logits, draft_logits, draft_tokens, uniforms, temperature, B, K, V, n_accepted,
                       next_token, workspace, workspace_bytes, stream, false);
}

sv_status sv_verify_sample_logits_early_batched(const float* target_logits, const float* draft_logits,
                                                const int32_t* draft_tokens, const float* uniforms,
                                                float temperature, int32_t B, int32_t K, int32_t V,
                                                int32_t* n_accepted, int32_t* next_token,
                                                void* workspace, size_t workspace_bytes, void* stream)
{
    return logits_call(target_logits, draft_logits, draft_tokens, uniforms, temperature, B, K, V, n_accepted,
                       next_token, workspace, workspace_bytes, stream, true);
}
}   // extern "C"

namespace {
sv_status logits_call(const float* target_logits, const float* draft_logits,
                      const int32_t* draft_tokens, const float* uniforms, float temperature,
                      int32_t B, int32_t K, int32_t V,
                      int32_t* n_accepted, int32_t* next_token,
                      void* workspace, size_t workspace_bytes, void* stream, bool early)
{
    sv_status st = check_sizes(B, K, V);
    if (st != SV_OK) return st;
    if (!(std::isfinite(temperature) && temperature > 0.0f)) return SV_ERR_INVALID_ARG;
    if (B == 0) return SV_OK;   // nothing to verify; pointers are not inspected
    if (!target_logits || !uniforms || !n_accepted || !next_token ||
        (K > 0 && (!draft_logits || !draft_tokens)))
        return SV_ERR_INVALID_ARG;
    if (!aligned(target_logits, 4) || !aligned(draft_logits, 4) || !aligned(draft_tokens, 4) ||
        !aligned(uniforms, 4) || !aligned(n_accepted, 4) || !aligned(next_token, 4))
        return SV_ERR_INVALID_ARG;
    if (!workspace || !aligned(workspace, 16) || workspace_bytes < sv_workspace_size(B, K, V, 1))
        return SV_ERR_WORKSPACE;
    DevInfo d;
    st = device_info(&d);
    if (st != SV_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Args a = make_args(workspace, B, K, V, true);
    st = next_epoch(workspace, workspace_bytes, s, &a.epoch);
    if (st != SV_OK) return st;
    a.tp = target_logits;
    a.dp = draft_logits;
    a.dt = draft_tokens;
    a.u = uniforms;
    a.n_out = n_accepted;
    a.next_out = next_token;
    // exp(x / tau) = exp2(x * log2(e) / tau)
    a.ktau64 = 1.4426950408889634 / (double)temperature;
    a.ktau = (float)a.ktau64;
    const Tuning tu = tuning();
    a.force_recompute = tu.force_recompute;
    a.force_lost = tu.force_lost;
    a.poll_ticks = (unsigned long long)(tu.poll_us * 1e-3 * (double)d.wall_khz);
    const bool vec = (V % 4 == 0) && aligned(target_logits, 16) && (K == 0 || aligned(draft_logits, 16));
    const uint64_t per_row = (uint64_t)B * (uint64_t)a.NC;
    const uint64_t bonus = (uint64_t)B * (uint64_t)((a.NC + kBonusChunks - 1) / kBonusChunks);
    const bool rows = use_rows(K, per_row, bonus, kRowsBlocksPerRowL, tu);
    a.nwalk = (unsigned)(K > 0 ? (rows ? (uint64_t)K * per_row : per_row) : 0);
    const dim3 grid((unsigned)(a.nwalk + bonus)), block(kThreads);
    a.early = early ? 1 : 0;
    if (vec && rows)
        hipLaunchKernelGGL((sv_logits_kernel<true, true>), grid, block, 0, s, a);
    else if (vec && early)
        hipLaunchKernelGGL((sv_logits_kernel<true, false, true>), grid, block, 0, s, a);
    else if (vec)
        hipLaunchKernelGGL((sv_logits_kernel<true, false>), grid, block, 0, s, a);
    else if (rows)
        hipLaunchKernelGGL((sv_logits_kernel<false, true>), grid, block, 0, s, a);
    else if (early)
        hipLaunchKernelGGL((sv_logits_kernel<false, false, true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((sv_logits_kernel<false, false>), grid, block, 0, s, a);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}
}   // namespace

extern "C" {

sv_status sv_workspace_error(const void* workspace, int32_t* error_out, void* stream)
{
    if (!workspace || !error_out) return SV_ERR_INVALID_ARG;
    if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return SV_ERR_HIP;
    unsigned v = 0;
    const unsigned char* w = static_cast<const unsigned char*>(workspace);
    if (hipMemcpy(&v, w + offsetof(Header, error), sizeof(v), hipMemcpyDeviceToHost) != hipSuccess)
        return SV_ERR_HIP;
    *error_out = (int32_t)v;
    return SV_OK;
}

const char* sv_status_string(sv_status s)
{
    switch (s) {
    case SV_OK: return "SV_OK";
    case SV_ERR_INVALID_ARG: return "SV_ERR_INVALID_ARG: NULL, misaligned or negative argument";
    case SV_ERR_WORKSPACE: return "SV_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case SV_ERR_HIP: return "SV_ERR_HIP: a HIP runtime call or kernel launch failed";
    case SV_ERR_UNSUPPORTED: return "SV_ERR_UNSUPPORTED: size beyond the supported maximum";
    case SV_ERR_SCRATCH: return "SV_ERR_SCRATCH: the call needs more than the static scratch (SV_SCRATCH_BYTES)";
    }
    return "unknown sv_status";
}

}  // extern "C"
