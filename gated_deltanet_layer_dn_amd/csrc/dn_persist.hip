// Whole-stack decode kernel for single-sequence stacks with 128x128 value-head state tiles.
//
// One launch runs one decode token through every layer of the stack (page "qwen36: run the
// DeltaNet layer end to end on the card", section "What the PR does", Backend paragraph: in_proj
// GEMV, conv + SiLU with the history advancing, per value head L2 norms with eps inside the sqrt,
// decay, delta rule against the decayed state, write-back, readout over the updated state, gated
// RMSNorm with silu(z), out_proj GEMV).
//
// Layout of the work. One workgroup per compute unit, each with eight compute waves and four
// communication waves.
//  * Phase A (in_proj + conv + SiLU): each workgroup owns a contiguous band of in_proj rows; each
//    compute wave streams RA of them. The rows' weights are loaded into registers one layer ahead,
//    as soon as the previous layer's phase A has used them, so the HBM stream never waits for the
//    activations.
//  * Phase B (recurrence): workgroup b owns value head b / (dv/16) and 16 of its value columns; its
//    first communication wave keeps that 128x16 slice of the state in registers (lane 4j+p: column
//    j, key rows 32p..32p+31), prefetched one layer ahead. It decays the slice, takes the sums
//    for the delta and for the readout over the updated state in one pass, publishes the gated
//    readout of its columns and only then writes the delta rule into the slice; sums over the key
//    rows are in-lane plus two DPP steps.
//  * Phase C (gated RMSNorm finish + out_proj): each workgroup owns D/NWG out_proj rows.
// Hand-offs between workgroups carry no fences: every cross-workgroup value travels in a tagged
// word stored and loaded with device-coherent (sc1) accesses, and a reader spins until each word
// carries the tag of the current layer and token. The in_proj output, which each reader gathers
// only in part, uses 64-bit words (fp32 value, 32-bit tag); the layer output and the gated readout,
// which every workgroup reads whole, use 32-bit words whose two low mantissa bits hold the tag mod
// 4, read four at a time. Tags grow by one per layer and never repeat within 2^32 layer steps, so
// buffers need no reset between launches (dn_set_state restarts them after an aborted launch).
// Compute waves never poll, so their outstanding weight prefetches never delay a hand-off (a
// wave's loads complete in order); the communication waves poll, stage activations into LDS, and
// run phase B. The next layer's in_proj rows are requested only after phase B's inputs arrived.
//
// GEMV arithmetic: activations split into three int8 terms, exact int32 dot products with
// v_dot4_i32_i8 per lane, folded into one fp32 partial per lane and summed over the wave in fp32.
//
// Gates on the card (GT): in every phase-B workgroup the second communication wave computes the
// in_proj rows of its head's two gates (R + bh and R + Hv + bh) on the staged x during phase A,
// applies the gate functions, and hands alpha and beta to phase B through LDS: no hand-off between
// workgroups for them (each head's gate rows are read by its eight workgroups).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "dn_internal.h"

namespace dn {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int NCW = 8;                 // compute waves per workgroup
constexpr int NCM = 4;                 // communication waves per workgroup
constexpr int NTHR = (NCW + NCM) * 64;
constexpr int DK = 128;                // key rows of a state tile
constexpr int CB = 16;                 // value columns per phase-B workgroup
constexpr int MAXL = 256;              // layers per handle (the C ABI's limit)
// Weight prefetch throttle: a compute wave keeps at most this many 1 KiB row-chunk loads in
// flight, so that the compute unit's memory pipeline is never full and the communication
// waves' hand-off loads and stores are not queued behind a whole layer of weights.
#ifndef DN_PREFETCH_INFLIGHT
#define DN_PREFETCH_INFLIGHT 3
#endif
static_assert(DN_PREFETCH_INFLIGHT >= 1 && DN_PREFETCH_INFLIGHT < 16, "");
// The last DN_PREFETCH_TAIL row-chunk loads of each part of a layer's in_proj prefetch are issued
// without the throttle.
#ifndef DN_PREFETCH_TAIL
#define DN_PREFETCH_TAIL 2
#endif
// A compute wave prefetches the first DN_PREFETCH_EARLY_ROWS of its in_proj rows of the next layer
// while phase B and the gated-readout exchange run, and the others after phase C (issuing them all
// before phase C kept the compute waves from phase C well after the readout had arrived).
#ifndef DN_PREFETCH_EARLY_ROWS
#define DN_PREFETCH_EARLY_ROWS 4
#endif

// s_waitcnt with vmcnt <= n and the other counters unconstrained
#define DN_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | (n))

// Instrumented builds (-DDN_PHASE_TIMERS) record the 100 MHz wall clock at phase boundaries of the
// first TS_MAXL layers into LDS (so that the instrumentation holds no registers across the phases)
// and copy them to PersistArgs::timers [NWG][L][32] when the launch ends.
#ifdef DN_PHASE_TIMERS
constexpr int TS_MAXL = 32;
__shared__ unsigned long long g_ts[TS_MAXL][32];
// the marks recorded (a bit per mark index); the others compile to nothing, which keeps the
// instrumented kernel's registers as the uninstrumented one's
#ifndef DN_TS_MARKS
#define DN_TS_MARKS ((1u << 1) | (1u << 2) | (1u << 3) | (1u << 4) | (1u << 15) | (1u << 6) | (1u << 7) | (1u << 8))
#endif
#define DN_MARK(a, l, k)                                                                              \
  do {                                                                                                \
    if (((DN_TS_MARKS) >> (k)) & 1u)                                                                  \
      if ((threadIdx.x & 63) == 0 && (l) < TS_MAXL) g_ts[(l)][(k)] = wall_clock64();                \
  } while (0)
#else
#define DN_MARK(a, l, k) \
  do {                   \
  } while (0)
#endif

__device__ __forceinline__ int sdot4(int a, int b, int c) { return __builtin_amdgcn_sdot4(a, b, c, false); }
__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }

__device__ __forceinline__ void ll_store(uint64_t* p, float v, unsigned tag) {
  const uint64_t w = ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v);
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ll_load(const __attribute__((address_space(1))) uint64_t* p) {
  return __hip_atomic_load(const_cast<__attribute__((address_space(1))) uint64_t*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned coherent_load_u32(const unsigned* p) {
  return __hip_atomic_load(const_cast<unsigned*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coherent_store_u32(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Self-tagged 32-bit hand-off words: the fp32 value rounded to nearest at 21 mantissa bits (relative
// change at most 2^-22), its two lowest bits replaced by the layer tag mod 4. Every reader of these
// buffers reads every word each layer, and no producer runs more than one layer ahead of a reader,
// so a word holds either the previous layer's tag or the current one: two bits tell them apart.
// Tearing between the words of a 16-byte load is harmless since each word carries its own tag.
__device__ __forceinline__ unsigned st_pack(float v, unsigned tag) {
  return ((__float_as_uint(v) + 2u) & ~3u) | (tag & 3u);
}
__device__ __forceinline__ float st_value(unsigned w) { return __uint_as_float(w & ~3u); }
__device__ __forceinline__ void st_store(unsigned* p, float v, unsigned tag) {
  __hip_atomic_store(p, st_pack(v, tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool st_tagged(const v4u& q, unsigned t) {
  return ((q[0] & 3u) == t) & ((q[1] & 3u) == t) & ((q[2] & 3u) == t) & ((q[3] & 3u) == t);
}
// Global-address-space view of a device pointer. Pointers read from the per-layer table (or passed
// through an empty asm statement) are generic to the compiler, which then emits flat loads; a flat
// load counts on the LDS counter as well as the vector-memory one, so every LDS wait of the wave
// (lgkmcnt(0), the workgroup barriers' included) would also wait for it. Through this view the
// weight prefetches and the in_proj polls are global loads, which LDS waits do not wait for.
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* gmem(const T* p) {
  return (const __attribute__((address_space(1))) T*)p;
}
// Buffer resource over `bytes` bytes at p (raw, untyped 32-bit accesses).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
constexpr int CPOL_SC1 = 16;  // cache policy of a device-coherent load (and store)
// A self-tagged word stored through a buffer resource at byte offset boff, with the same
// device-coherent write-through policy as the agent-scope atomic store above: the address is a
// 32-bit offset from a scalar base instead of a 64-bit register pair per lane.
__device__ __forceinline__ void st_store_rs(__amdgpu_buffer_rsrc_t rs, int boff, float v, unsigned tag) {
  __builtin_amdgcn_raw_buffer_store_b32(st_pack(v, tag), rs, boff, 0, CPOL_SC1);
}


// Staged activation position of column c (4-bit weights hold 8 columns per dword as nibbles;
// the masked low and high nibbles are the even and odd columns).
template <int BITS>
__device__ __forceinline__ int xpos(int c) {
  if (BITS == 8) return c;
  return (c & ~7) | ((c & 1) << 2) | ((c >> 1) & 3);
}

// One term of the int8 split: q = rint(r inv) clamped to [-127, 127] (v_med3), found by adding
// 1.5 * 2^23, which rounds to an integer (ties to even) and leaves it, two's complement, in the low
// mantissa bits: the returned word's low byte is the int8 term, and q is that word minus the bias.
constexpr float SPLIT_BIAS = 12582912.0f;
__device__ __forceinline__ unsigned split_term(float r, float inv, float& q) {
  const float t = __builtin_amdgcn_fmed3f(r * inv, -127.0f, 127.0f) + SPLIT_BIAS;
  q = t - SPLIT_BIAS;
  return __float_as_uint(t);
}
// The low bytes of four words, word i into byte i.
__device__ __forceinline__ unsigned low_bytes(unsigned w0, unsigned w1, unsigned w2, unsigned w3) {
  const unsigned lo = __builtin_amdgcn_perm(w1, w0, 0x0c0c0400u);  // w0.b0, w1.b0, 0, 0
  const unsigned hi = __builtin_amdgcn_perm(w3, w2, 0x0c0c0400u);
  return lo | (hi << 16);
}


// Dot products of RB rows (NCH 16-byte chunks per lane each) with the staged three-term
// activations in LDS. acc[i][t] gets lane partial sums of term t for row i.
template <int BITS, int RB, int NCH>
__device__ __forceinline__ void dot_rows(const v4i (&w)[RB][NCH], const int8_t* xs, int cols, int lane,
                                         int (&acc)[RB][3]) {
#pragma unroll
  for (int i = 0; i < RB; ++i) acc[i][0] = acc[i][1] = acc[i][2] = 0;
  const v4i* X0 = reinterpret_cast<const v4i*>(xs);
  const v4i* X1 = reinterpret_cast<const v4i*>(xs + cols);
  const v4i* X2 = reinterpret_cast<const v4i*>(xs + 2 * cols);
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int c = lane + 64 * k;
    if (BITS == 8) {
      const v4i x0 = X0[c], x1 = X1[c], x2 = X2[c];
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[i][0] = sdot4(w[i][k][e], x0[e], acc[i][0]);
          acc[i][1] = sdot4(w[i][k][e], x1[e], acc[i][1]);
          acc[i][2] = sdot4(w[i][k][e], x2[e], acc[i][2]);
        }
    } else {
      const v4i a0 = X0[2 * c], b0 = X0[2 * c + 1], a1 = X1[2 * c], b1 = X1[2 * c + 1];
      const v4i a2 = X2[2 * c], b2 = X2[2 * c + 1];
      const int e0[4] = {a0[0], a0[2], b0[0], b0[2]}, o0[4] = {a0[1], a0[3], b0[1], b0[3]};
      const int e1[4] = {a1[0], a1[2], b1[0], b1[2]}, o1[4] = {a1[1], a1[3], b1[1], b1[3]};
      const int e2[4] = {a2[0], a2[2], b2[0], b2[2]}, o2[4] = {a2[1], a2[3], b2[1], b2[3]};
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // signed nibbles moved to the high half of each byte: bytes hold 16 * w
          const unsigned p = (unsigned)w[i][k][e];
          const int lo = (int)((p << 4) & 0xF0F0F0F0u), hi = (int)(p & 0xF0F0F0F0u);
          acc[i][0] = sdot4(hi, o0[e], sdot4(lo, e0[e], acc[i][0]));
          acc[i][1] = sdot4(hi, o1[e], sdot4(lo, e1[e], acc[i][1]));
          acc[i][2] = sdot4(hi, o2[e], sdot4(lo, e2[e], acc[i][2]));
        }
    }
  }
}

// LDS of a workgroup. HB: communication waves that run phase B (1: a 128 x 16 state slice per
// workgroup; 2: a 128 x 32 slice in two halves, for up to 64 value heads, with the out_proj rows
// prefetched into LDS rather than registers to make room for 8 in_proj rows per compute wave).
// LDS only the two-wave form uses (empty, and so of no size, for HB == 1)
template <int HB>
struct SmemB2 {};
template <>
struct SmemB2<2> {
  int v_ready;             // layers whose second-half v, z are in vz
  float vz[2 * CB];        // v and z of the second half's columns
  v4i wcl[8 * 8 * 64];     // the out_proj row of each compute wave, [wave][chunk][lane]
};
template <int HB, int DKT = DK>
struct SmemT : SmemB2<HB> {
  static constexpr int VMAX = HB == 1 ? 4096 : 8192;  // readout columns
#ifdef DN_PHASE_TIMERS
  static constexpr int LMAX = HB == 1 ? MAXL : 32;    // (the instrumented build's marks take 8 KB of LDS)
#else
  static constexpr int LMAX = HB == 1 ? MAXL : 64;    // layers whose per-layer tables are held
#endif
  float raw[4096];         // staged layer input x, fp32
  float yf[VMAX];          // gated, normalised readout y (input of out_proj), fp32
  int8_t xs[3 * 4096];     // three-term split of x for phase A
  float inv[64];           // per value head 1/rms of the readout
  float qk[2 * DKT];       // raw q and k of phase B's key head
  v4i gwl[2][2][64];       // GT: the next layer's two gate rows of this head (lane's 16-byte chunks), via LDS DMA
  float gval[2];           // GT: the layer's gates alpha, beta of this head
  v4f sbuf[HB][DKT / 16 * 64];  // phase B's updated state slice until its write-back (HB halves of 16 columns)
  float stat[16];          // partial statistics from the communication waves, split scale
  float gate[LMAX][2];     // alpha, beta of this workgroup's value head, per layer
  float nw[LMAX][HB * CB]; // gated RMSNorm weights of this workgroup's value columns, per layer
  int a_done, b_done, c_done;  // progress counters of this workgroup's waves
  int u_done;                  // phase-B inputs received (the next layer's in_proj prefetch may start)
  int s_ready;                 // compute waves whose chunk of the layer's state slice is in LDS
  int g_ready;                 // GT: layers whose gate values are in gval
  int abort_flag;
};
using Smem = SmemT<1>;

// Position in Smem::yf of readout column c: phase C reads, for lane l and 16-byte weight chunk k,
// the readout quads of the chunk's columns as one contiguous 16-byte word per lane, so that the
// wave's LDS reads are consecutive rather than 64 bytes apart (8-bit weights: 16 columns per chunk,
// 4-bit: 32).
template <int BITS>
__device__ __forceinline__ int ypos(int c) {
  constexpr int CWC = BITS == 8 ? 16 : 32, NQ = CWC / 4;
  const int l = (c / CWC) & 63, k = c / (64 * CWC), q = (c % CWC) >> 2;
  return ((k * NQ + q) * 64 + l) * 4 + (c & 3);
}

// Workgroup barrier for the per-layer hand-over of LDS data between the two wave roles. Unlike
// __syncthreads(), whose fence waits for every outstanding global access of the wave (loads
// included), it waits only for this wave's LDS accesses: the compute waves' weight prefetches stay
// in flight across it. No global data passes between the waves of a workgroup through these
// barriers (the hand-offs carry their own tags, and the state slice's copy into LDS is waited for
// explicitly).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait (within the workgroup) until an LDS progress counter reaches `target` or the workgroup
// aborts. The waves that advance the counter never wait on the waiting wave, so this ends.
__device__ __forceinline__ void wait_counter(const int* ctr, int target, const int* abort_flag) {
  while (__hip_atomic_load(const_cast<int*>(ctr), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target &&
         !__hip_atomic_load(const_cast<int*>(abort_flag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP))
    __builtin_amdgcn_s_sleep(1);
}
__device__ __forceinline__ int bump_counter(int* ctr) {
  return __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Replicas of the broadcast hand-off buffers: producers write one copy per XCD and each consumer
// reads the copy of its own XCD, so a polled line is shared by the 32 workgroups of one XCD
// rather than by all 256.
constexpr int NREP = 8;
__device__ __forceinline__ int xcd_id() { return (int)(__builtin_amdgcn_s_getreg((20) | (0 << 6) | (3 << 11)) & 7); }

// Sum over the 64 lanes of a wave with DPP lane permutations (pairs, quads, half rows, rows,
// then across rows); the total is returned uniformly. Fixed order: run-to-run identical.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}
__device__ __forceinline__ float wave_total_f(float x) {
  int v = __float_as_int(x);
  v = __float_as_int(__int_as_float(v) + __int_as_float(dpp_i<0xB1>(v)));
  v = __float_as_int(__int_as_float(v) + __int_as_float(dpp_i<0x4E>(v)));
  v = __float_as_int(__int_as_float(v) + __int_as_float(dpp_i<0x141>(v)));
  v = __float_as_int(__int_as_float(v) + __int_as_float(dpp_i<0x140>(v)));
  v = __float_as_int(__int_as_float(v) + __int_as_float(dpp_i<0x142, 0xA>(v)));
  v = __float_as_int(__int_as_float(v) + __int_as_float(dpp_i<0x143, 0xC>(v)));
  return __int_as_float(__builtin_amdgcn_readlane(v, 63));
}

__device__ __forceinline__ double wave_total_d(double x) {
#define DN_DPP_D(CTRL, RM)                                                                          \
  x += __hiloint2double(dpp_i<CTRL, RM>(__double2hiint(x)), dpp_i<CTRL, RM>(__double2loint(x)))
  DN_DPP_D(0xB1, 0xF);
  DN_DPP_D(0x4E, 0xF);
  DN_DPP_D(0x141, 0xF);
  DN_DPP_D(0x140, 0xF);
  DN_DPP_D(0x142, 0xA);
  DN_DPP_D(0x143, 0xC);
#undef DN_DPP_D
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(x), 63),
                          __builtin_amdgcn_readlane(__double2loint(x), 63));
}
// Sum over each group of four consecutive lanes; all four receive the same total.
__device__ __forceinline__ float quad_sum(float x) {
  x += __int_as_float(dpp_i<0xB1>(__float_as_int(x)));
  x += __int_as_float(dpp_i<0x4E>(__float_as_int(x)));
  return x;
}
// Sum over each group of eight consecutive lanes (quads, then the mirrored half row).
__device__ __forceinline__ float oct_sum(float x) {
  x = quad_sum(x);
  x += __int_as_float(dpp_i<0x141>(__float_as_int(x)));
  return x;
}
// Maximum over the 64 lanes of a wave (of non-negative values) with DPP lane permutations,
// returned uniformly.
__device__ __forceinline__ float wave_max_f(float x) {
  int v = __float_as_int(x);
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp_i<0xB1>(v))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp_i<0x4E>(v))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp_i<0x141>(v))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp_i<0x140>(v))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp_i<0x142, 0xA>(v))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp_i<0x143, 0xC>(v))));
  return __int_as_float(__builtin_amdgcn_readlane(v, 63));
}

// Reduce the lane partials of RB rows; lane i (< RB) receives row i's dot product. Each lane's three
// term sums are exact integers below 2^24 (so exact in fp32); they are folded into one fp32 partial
// per lane, v ~= s1 (h + (m + l/254)/254), and each row takes one fp32 wave sum (three integer
// wave sums per row, folded in double, measured 5.7 us per token slower on the 30-layer stack).
template <int BITS, int RB>
__device__ __forceinline__ float reduce_rows(int (&acc)[RB][3], float s1, int lane) {
  float mine = 0.f;
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    const float f = fmaf(fmaf((float)acc[i][2], 1.0f / 254.0f, (float)acc[i][1]), 1.0f / 254.0f, (float)acc[i][0]);
    const float d = wave_total_f(f) * (BITS == 4 ? s1 * (1.0f / 16.0f) : s1);  // nibble products carry 16
    if (lane == i) mine = d;
  }
  return mine;
}

// Poll N 64-bit tagged words per lane, word i at base + off[i] (element offsets), until every one
// carries `want`; values go to v[]. Returns false after `cap` rounds, or if another workgroup
// reported an error. The base pointer is laundered through an empty asm statement each round so
// that the compiler rebuilds the addresses from one register pair with immediate offsets instead
// of keeping N 64-bit addresses alive across the loop.
template <int N>
__device__ __forceinline__ bool poll_words_at(const uint64_t* base, const int (&off)[N], unsigned want, float (&v)[N],
                                              unsigned nvalid, const unsigned* err, unsigned cap,
                                              unsigned* rounds = nullptr) {
  unsigned pend = (1u << N) - 1u;
  pend &= (1u << nvalid) - 1u;
  unsigned it = 0;
  while (__any(pend != 0)) {
    const __attribute__((address_space(1))) uint64_t* b = gmem(base);
    asm volatile("" : "+v"(b));
    uint64_t w[N];
#pragma unroll
    for (int i = 0; i < N; ++i)
      if ((pend >> i) & 1) w[i] = ll_load(b + off[i]);
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (((pend >> i) & 1) && (unsigned)(w[i] >> 32) == want) {
        v[i] = __uint_as_float((unsigned)w[i]);
        pend &= ~(1u << i);
      }
    if (++it > cap || ((it & 255) == 0 && coherent_load_u32(err))) return false;
  }
  if (rounds) *rounds = it;
  return true;
}

// Poll NQ 16-byte quads of self-tagged words per lane, quad i at byte offset boff + i * QSTRIDE of
// the buffer, with device-coherent loads until every word carries `want` mod 4; quads i >= nvalid
// are not polled. When ONE is set, the single word at byte offset boff1 is polled as well. Returns
// false after `cap` rounds, or if another workgroup reported an error.
template <int NQ, int QSTRIDE, int NX>
__device__ __forceinline__ bool poll_quads(__amdgpu_buffer_rsrc_t rs, int boff, int boff1, unsigned want, v4u (&q)[NQ],
                                           unsigned (&w1)[2], const unsigned* err, unsigned cap) {
  static_assert(NX >= 0 && NX <= 2, "");
  const unsigned t = want & 3u;
  unsigned pend = (1u << NQ) - 1u;
  bool pend1 = NX > 0;
  unsigned it = 0;
  typedef unsigned v2u __attribute__((ext_vector_type(2)));
  while (__any((pend != 0) | pend1)) {
#pragma unroll
    for (int i = 0; i < NQ; ++i)
      if ((pend >> i) & 1)
        q[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, boff + i * QSTRIDE, 0, CPOL_SC1);
    if (NX == 1 && pend1) w1[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, boff1, 0, CPOL_SC1);
    if (NX == 2 && pend1) {
      const v2u p = __builtin_amdgcn_raw_buffer_load_b64(rs, boff1, 0, CPOL_SC1);
      w1[0] = p[0];
      w1[1] = p[1];
    }
#pragma unroll
    for (int i = 0; i < NQ; ++i)
      if (((pend >> i) & 1) && st_tagged(q[i], t)) pend &= ~(1u << i);
    if (NX == 1 && pend1 && (w1[0] & 3u) == t) pend1 = false;
    if (NX == 2 && pend1 && (w1[0] & 3u) == t && (w1[1] & 3u) == t) pend1 = false;
    if (++it > cap || ((it & 255) == 0 && coherent_load_u32(err))) return false;
  }
  return true;
}

// Work split shared by both wave roles.
struct Geo {
  int a_per_wg;
  int a_row0, a_row_end, c_row0, c_row_end;
  bool has_b;
  int bh, bcb, bg;
};

template <int BITS, int D, typename SM>
__device__ __forceinline__ void split_x(SM& sm, const PersistArgs& a, int tid) {
  // Three-term int8 split of the raw x with s1 = max|x| / 127: x ~= s1 (h + (m + l/254)/254); the
  // RMS factor joins s1 in the fold of the dot products (sm.stat[8]). Each thread splits 8
  // consecutive columns and writes each term as two dwords (4-bit weights: even columns in the
  // first, odd in the second, the staged order of xpos).
  constexpr int NT = D / 8;
  const float ss = (sm.stat[0] + sm.stat[1]) + (sm.stat[2] + sm.stat[3]);
  const float mx = fmaxf(fmaxf(sm.stat[4], sm.stat[5]), fmaxf(sm.stat[6], sm.stat[7]));
  const float scale = (a.flags & DN_X_RMSNORM) ? rsqrtf(ss / (float)D + a.eps_rms) : 1.0f;
  float s1 = mx * (1.0f / 127.0f);
  if (!(s1 > 0.f)) s1 = 1.0f;
  if (tid == 0) sm.stat[8] = s1 * scale;
  if (tid >= NT) return;
  const float inv1 = 1.0f / s1, s2 = s1 * (1.0f / 254.0f), inv2 = inv1 * 254.0f, inv3 = inv2 * 254.0f;
  for (int t = tid; t < NT; t += NTHR) {
    const v4f r0 = *reinterpret_cast<const v4f*>(sm.raw + 8 * t), r1 = *reinterpret_cast<const v4f*>(sm.raw + 8 * t + 4);
    const float v[8] = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
    unsigned wh[8], wm[8], wl[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float h, m, l;
      wh[e] = split_term(v[e], inv1, h);
      const float rr1 = fmaf(-s1, h, v[e]);
      wm[e] = split_term(rr1, inv2, m);
      const float rr2 = fmaf(-s2, m, rr1);
      wl[e] = split_term(rr2, inv3, l);
    }
    // staged column order: identity for 8-bit weights; for 4-bit the even columns, then the odd
    constexpr int o0 = 0, o1 = BITS == 8 ? 1 : 2, o2 = BITS == 8 ? 2 : 4, o3 = BITS == 8 ? 3 : 6;
    constexpr int o4 = BITS == 8 ? 4 : 1, o5 = BITS == 8 ? 5 : 3, o6 = BITS == 8 ? 6 : 5, o7 = 7;
    typedef unsigned v2u __attribute__((ext_vector_type(2)));
    *reinterpret_cast<v2u*>(sm.xs + 8 * t) = v2u{low_bytes(wh[o0], wh[o1], wh[o2], wh[o3]), low_bytes(wh[o4], wh[o5], wh[o6], wh[o7])};
    *reinterpret_cast<v2u*>(sm.xs + D + 8 * t) = v2u{low_bytes(wm[o0], wm[o1], wm[o2], wm[o3]), low_bytes(wm[o4], wm[o5], wm[o6], wm[o7])};
    *reinterpret_cast<v2u*>(sm.xs + 2 * D + 8 * t) = v2u{low_bytes(wl[o0], wl[o1], wl[o2], wl[o3]), low_bytes(wl[o4], wl[o5], wl[o6], wl[o7])};
  }
}

// Compute waves: phase A and phase C, weights prefetched one layer ahead in registers. (PK and GT
// do not change this role; they keep one specialisation per kernel instantiation, which the host
// compiler pass needs when several instantiations of the kernel are referenced.)
template <int BITS, int NCHA, int NCHC, int RA, int RC, bool PK, bool GT, int HB, int DKT>
__device__ __forceinline__ void compute_role(SmemT<HB, DKT>& sm, const PersistArgs& a, const Geo& g, unsigned base_tag,
                                             const float* S_in, float* S_out, const float* ring_in, float* ring_out,
                                             int tid, int lane) {
  constexpr int COLS_PER_CHUNK = BITS == 8 ? 1024 : 2048;
  constexpr int D = COLS_PER_CHUNK * NCHA, V = COLS_PER_CHUNK * NCHC;
  constexpr int rowbytes_in = BITS == 8 ? D : D / 2;
  constexpr int rowbytes_out = BITS == 8 ? V : V / 2;
  const int C = a.C, K = a.K;
  // HB == 2: the out_proj row (RC == 1) is prefetched into LDS (sm.wcl) with direct-to-LDS loads,
  // not into registers; wc then only carries a chunk at a time through phase C
  constexpr bool WCL = HB == 2;
  static_assert(!WCL || RC == 1, "");
  v4i wa[RA][NCHA];
  v4i wc[RC][WCL ? 1 : NCHC];
  const int cwv = tid >> 6;
  float ra_s = 0.f, ra_cw[4] = {0.f, 0.f, 0.f, 0.f}, ra_ring[3] = {0.f, 0.f, 0.f};
  float rc_s = 0.f;

  // in_proj rows of layer l into registers: part 0 the first DN_PREFETCH_EARLY_ROWS rows (and the
  // rows' scales, conv taps and history), part 1 the others; each part throttled to
  // DN_PREFETCH_INFLIGHT loads in flight but for its last DN_PREFETCH_TAIL
  // (with more rows per wave than 6, the extra ones join part 0: part 1 keeps its two rows)
  constexpr int EARLY0 = DN_PREFETCH_EARLY_ROWS + (RA > 6 ? RA - 6 : 0);
  constexpr int EARLY = EARLY0 < RA ? EARLY0 : RA;
  auto load_a = [&](int l, int part) {
    const LayerW& W = a.layers[l];
    const int8_t* wbase = reinterpret_cast<const int8_t*>(W.w_in);
#pragma unroll
    for (int i = 0; i < RA; ++i) {
      if ((part == 0) != (i < EARLY)) continue;
      const int r = g.a_row0 + i;
#pragma unroll
      for (int k = 0; k < NCHA; ++k) {
        const int n = (part == 0 ? i : i - EARLY) * NCHA + k, ntot = (part == 0 ? EARLY : RA - EARLY) * NCHA;
        if (n >= DN_PREFETCH_INFLIGHT && n < ntot - DN_PREFETCH_TAIL) DN_WAIT_VMCNT(DN_PREFETCH_INFLIGHT - 1);
        if (r < g.a_row_end)
          wa[i][k] = __builtin_nontemporal_load(gmem(reinterpret_cast<const v4i*>(wbase + (size_t)r * rowbytes_in) + lane + 64 * k));
        else
          wa[i][k] = v4i{0, 0, 0, 0};
      }
    }
    if (part != 0) return;
    int ln = lane;
    if constexpr (HB == 2) asm volatile("" : "+v"(ln));  // (recomputed here rather than held: it spilled)
    const int r = g.a_row0 + ln;
    if (lane < RA && r < g.a_row_end) {
      ra_s = *gmem(W.s_in + r);
      if (r < C) {
        const auto cwp = gmem(W.conv_w + (size_t)r * K);
        const auto rg = gmem(ring_in + (size_t)l * (K - 1) * C + r);
#pragma unroll
        for (int j = 0; j < 4; ++j) ra_cw[j] = j < K ? cwp[j] : 0.f;
#pragma unroll
        for (int j = 0; j < 3; ++j) ra_ring[j] = j < K - 1 ? rg[(size_t)j * C] : 0.f;
      }
    }
  };
  auto load_c = [&](int l) {
    const LayerW& W = a.layers[l];
    const int8_t* wbase = reinterpret_cast<const int8_t*>(W.w_out);
#pragma unroll
    for (int i = 0; i < RC; ++i) {
      // (HB == 2: the row index as a scalar, the wave's rows being uniform, so that the row's base
      // address is not held per lane)
      const int r = HB == 2 ? __builtin_amdgcn_readfirstlane(g.c_row0 + i) : g.c_row0 + i;
#pragma unroll
      for (int k = 0; k < NCHC; ++k) {
        if ((i * NCHC + k) >= DN_PREFETCH_INFLIGHT) DN_WAIT_VMCNT(DN_PREFETCH_INFLIGHT - 1);
        if constexpr (WCL) {
          // the previous layer's phase C read these slots: its LDS reads are done before they refill
          if (k == 0) __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
          if (r < g.c_row_end)
            __builtin_amdgcn_global_load_lds(gmem(reinterpret_cast<const v4i*>(wbase + (size_t)r * rowbytes_out) + lane + 64 * k),
                                             &sm.wcl[(cwv * 8 + k) * 64], 16, 0, 0);
          else
            sm.wcl[(cwv * 8 + k) * 64 + lane] = v4i{0, 0, 0, 0};
        } else {
          if (r < g.c_row_end)
            wc[i][WCL ? 0 : k] = __builtin_nontemporal_load(gmem(reinterpret_cast<const v4i*>(wbase + (size_t)r * rowbytes_out) + lane + 64 * k));
          else
            wc[i][WCL ? 0 : k] = v4i{0, 0, 0, 0};
        }
      }
    }
    const int r = g.c_row0 + lane;
    if (lane < RC && r < g.c_row_end) rc_s = *gmem(W.s_out + r);
  };

  // Phase B's state slice: compute wave w moves chunk w (lane's 4 floats at rows 32p + 4w, column
  // j, for lane 4j + p) between HBM and LDS: prefetched into LDS one layer ahead by a direct-to-LDS
  // load from the current state buffer, written back from LDS after phase C into the other one.
  // (HB == 2: chunk w of each half; the halves are 16 columns, CB * DK floats, apart)
  // (DKT = 256: each lane of a phase-B wave holds 64 key rows, and each compute wave moves two chunks,
  // cwv and cwv + 8, 32 floats apart)
  constexpr int RPL = DKT / 4, NCP = DKT / 128;
  const size_t s_off = ((size_t)g.bh * DKT + g.bcb * CB + (lane >> 2)) * DKT + RPL * (lane & 3) + 4 * cwv;
  // HB == 2: the same offset recomputed at each use from a laundered lane index (held across the
  // layers, it and the addresses built on it were spilled)
  auto soff = [&]() -> size_t {
    if constexpr (HB == 2) {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      return ((size_t)g.bh * DKT + g.bcb * CB + (ln >> 2)) * DKT + RPL * (ln & 3) + 4 * cwv;
    } else {
      return s_off;
    }
  };
  const size_t s_layer = (size_t)a.Hv * DKT * DKT;
  if (g.has_b) {
#pragma unroll
    for (int h = 0; h < HB; ++h)
#pragma unroll
      for (int c = 0; c < NCP; ++c)
        __builtin_amdgcn_global_load_lds(S_in + s_off + (size_t)h * CB * DKT + 32 * c, &sm.sbuf[h][64 * (cwv + 8 * c)], 16, 0, 0);
  }
  load_a(0, 0);
  load_a(0, 1);
  load_c(0);
  for (int l = 0; l < a.L; ++l) {
    const unsigned tag = base_tag + (unsigned)l;
    lds_barrier();  // (1) raw x staged
    if (sm.abort_flag) break;
    split_x<BITS, D>(sm, a, tid);
    lds_barrier();  // (2) x split staged
    if (tid == 0) DN_MARK(a, l, 2);
    {
      // phase A: in_proj + conv + SiLU
      const float s1 = sm.stat[8];
      int acc[RA][3];
      dot_rows<BITS, RA, NCHA>(wa, sm.xs, D, lane, acc);
      const float dot = reduce_rows<BITS, RA>(acc, s1, lane);
      if (g.has_b) {
        // this wave's chunk of the state slice has landed in LDS, before this phase's stores go
        // out (vector memory operations complete in order, stores included): the only operations
        // issued after its copy are the out_proj prefetch loads of this layer, RC * NCHC weight
        // loads and one scale load when the wave owns a row, none otherwise
        static_assert(RC * NCHC <= 15, "");
        if (g.c_row0 + RC <= g.c_row_end) DN_WAIT_VMCNT(RC * NCHC);
        else DN_WAIT_VMCNT(0);
        if (lane == 0) bump_counter(&sm.s_ready);
      }
      const int r = g.a_row0 + lane;
      if (lane < RA && r < g.a_row_end) {
        const float u = ra_s * dot;
        float outv = u;
        if (r < C) {
          float accv = ra_cw[K - 1] * u;
#pragma unroll
          for (int j = 0; j < 3; ++j)
            if (j < K - 1) accv = fmaf(ra_cw[j], ra_ring[j], accv);
          outv = silu(accv);
        }
        // the hand-off word first: stores leave in order, and the history's can wait
        ll_store(a.U + r, outv, tag);
        if (r < C) {
          float* rg = ring_out + (size_t)l * (K - 1) * C + r;
#pragma unroll
          for (int j = 0; j < 2; ++j)
            if (j + 1 < K - 1) rg[(size_t)j * C] = ra_ring[j + 1];
          if (K > 1) rg[(size_t)(K - 2) * C] = u;
        }
      }
      if (lane == 0) bump_counter(&sm.a_done);
      if (tid == 0) DN_MARK(a, l, 3);
      // the next layer's in_proj rows stream in once this workgroup's phase-B inputs have
      // arrived, so that the u hand-off is not queued behind them
      wait_counter(&sm.u_done, l + 1, &sm.abort_flag);
      if (l + 1 < a.L) load_a(l + 1, 0);
      if (tid == 0) DN_MARK(a, l, 28);
    }
    lds_barrier();  // (3) gated readout staged
    if (sm.abort_flag) break;
    if (tid == 0) DN_MARK(a, l, 7);
    {
      // phase C: out_proj in fp32 on the staged readout. Weight bytes are biased to unsigned
      // (w + 128, or w + 8 for nibbles) for the byte conversions; the bias times sum(y) is
      // removed after the row sum.
      const float sumy = (sm.stat[9] + sm.stat[10]) + (sm.stat[11] + sm.stat[12]);
      float acc[RC];
#pragma unroll
      for (int i = 0; i < RC; ++i) acc[i] = 0.f;
      const v4f* Y4 = reinterpret_cast<const v4f*>(sm.yf);
      if constexpr (WCL) {
        // the row's direct-to-LDS loads were issued before every load still in flight
        DN_WAIT_VMCNT(0);
        asm volatile("" ::: "memory");
      }
#pragma unroll
      for (int k = 0; k < NCHC; ++k) {
        if constexpr (WCL) wc[0][0] = sm.wcl[(cwv * 8 + k) * 64 + lane];
        if (BITS == 8) {
          const v4f yq[4] = {Y4[(k * 4 + 0) * 64 + lane], Y4[(k * 4 + 1) * 64 + lane], Y4[(k * 4 + 2) * 64 + lane],
                             Y4[(k * 4 + 3) * 64 + lane]};
#pragma unroll
          for (int i = 0; i < RC; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const unsigned u = (unsigned)wc[i][WCL ? 0 : k][e] ^ 0x80808080u;
              acc[i] = fmaf((float)(u & 0xFFu), yq[e][0], acc[i]);
              acc[i] = fmaf((float)((u >> 8) & 0xFFu), yq[e][1], acc[i]);
              acc[i] = fmaf((float)((u >> 16) & 0xFFu), yq[e][2], acc[i]);
              acc[i] = fmaf((float)(u >> 24), yq[e][3], acc[i]);
            }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // columns 32c + 8e .. +7 of the lane's chunk c = lane + 64 k
            const v4f ya = Y4[(k * 8 + 2 * e) * 64 + lane], yb = Y4[(k * 8 + 2 * e + 1) * 64 + lane];
#pragma unroll
            for (int i = 0; i < RC; ++i) {
              const unsigned p = (unsigned)wc[i][WCL ? 0 : k][e] ^ 0x88888888u;
              const unsigned lo = p & 0x0F0F0F0Fu, hi = (p >> 4) & 0x0F0F0F0Fu;
              acc[i] = fmaf((float)(lo & 0xFFu), ya[0], acc[i]);
              acc[i] = fmaf((float)(hi & 0xFFu), ya[1], acc[i]);
              acc[i] = fmaf((float)((lo >> 8) & 0xFFu), ya[2], acc[i]);
              acc[i] = fmaf((float)((hi >> 8) & 0xFFu), ya[3], acc[i]);
              acc[i] = fmaf((float)((lo >> 16) & 0xFFu), yb[0], acc[i]);
              acc[i] = fmaf((float)((hi >> 16) & 0xFFu), yb[1], acc[i]);
              acc[i] = fmaf((float)(lo >> 24), yb[2], acc[i]);
              acc[i] = fmaf((float)(hi >> 24), yb[3], acc[i]);
            }
          }
        }
      }
      float mine = 0.f;
#pragma unroll
      for (int i = 0; i < RC; ++i) {
        const float tot = wave_total_f(acc[i]) - (BITS == 8 ? 128.0f : 8.0f) * sumy;
        if (lane == i) mine = tot;
      }
      const int r = g.c_row0 + lane;
      const float o = rc_s * mine;
      if (l + 1 < a.L) {
        // lanes 0..NREP-1 write the replicas of each row, row i's value taken from lane i; these
        // hand-off words go out before the layer's output store
#pragma unroll
        for (int i = 0; i < RC; ++i) {
          const float oi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(o), i));
          const int ri = g.c_row0 + i;
          if (lane < NREP && ri < g.c_row_end) {
            if constexpr (HB == 2) {
              // through a buffer resource, the offset computed here from a laundered lane index
              // rather than held in a register across the layers (which spilled it)
              int ln = lane;
              asm volatile("" : "+v"(ln));
              st_store_rs(buf_rsrc(a.X, 4u * NREP * D), 4 * (ln * D + ri), oi, tag);
            } else
              st_store(a.X + (size_t)lane * D + ri, oi, tag);
          }
        }
      }
      if (lane < RC && r < g.c_row_end) a.out[(size_t)l * D + r] = o;
      if (lane == 0) bump_counter(&sm.c_done);
      if (tid == 0) DN_MARK(a, l, 8);
      if (g.has_b) {
        // write back this wave's chunk of the updated slice (parked in LDS by phase B before
        // barrier 3), then prefetch the next layer's chunk into the same LDS slots
        const size_t so = soff();
#pragma unroll
        for (int h = 0; h < HB; ++h)
#pragma unroll
          for (int c = 0; c < NCP; ++c) {
            const v4f v = sm.sbuf[h][64 * (cwv + 8 * c) + lane];
            *reinterpret_cast<v4f*>(S_out + (size_t)l * s_layer + so + (size_t)h * CB * DKT + 32 * c) = v;
          }
        if (l + 1 < a.L) {
          __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the LDS read is done before the slots refill
#pragma unroll
          for (int h = 0; h < HB; ++h)
#pragma unroll
            for (int c = 0; c < NCP; ++c)
              __builtin_amdgcn_global_load_lds(S_in + (size_t)(l + 1) * s_layer + so + (size_t)h * CB * DKT + 32 * c,
                                               &sm.sbuf[h][64 * (cwv + 8 * c)], 16, 0, 0);
        }
      }
      if (l + 1 < a.L) {
        load_c(l + 1);
        load_a(l + 1, 1);
      }
    }
  }
}

// Communication waves: poll and stage x and the gated readout; the first one also runs phase B.
// The polls of the layer input and of the gated readout start only once this workgroup's own
// share of that data is done, so that the rounds that are bound to miss are not issued (starting
// them at once measured slower); the in_proj poll of the recurrence starts at once.
// PK: one decay per key channel; apk [L][128] holds this head's decays (LDS).
// GT: gates from the in_proj's gate rows; sm.gate holds this head's a_log, a_bias per layer.
template <int BITS, int NCHA, int NCHC, bool PK, bool GT, int HB, int DKT>
__device__ __forceinline__ void comm_role(SmemT<HB, DKT>& sm, float (*apk)[DK], const PersistArgs& a, const Geo& g,
                                          unsigned base_tag, int tid, int lane, int cw, int wg) {
  constexpr int COLS_PER_CHUNK = BITS == 8 ? 1024 : 2048;
  constexpr int D = COLS_PER_CHUNK * NCHA, V = COLS_PER_CHUNK * NCHC, DV = DKT;  // (dv = dk)
  constexpr int XW = D / (64 * NCM);  // x words per lane
  constexpr int GW = V / (64 * NCM);  // gated readout words per lane
  constexpr int nblk = DV / CB;
  // words per communication wave segment of the G buffer: V/NCM readout columns, then the norm
  // partials of those heads (up to 64 HB of them: HB per lane in the staging)
  constexpr int GSEG = V / NCM + 64 * HB;
  constexpr int XQ = XW / 4, GQ = GW / 4;  // 16-byte quads per lane
  static_assert(XW % 4 == 0 && GW % 4 == 0 && XQ <= 4 && GQ <= 8, "");
  static_assert(HB == 1 || (HB == 2 && !GT && !PK && DKT == 128), "");
  static_assert(DKT == 128 || (DKT == 256 && HB == 1 && !GT && !PK), "");
  // phase B: q and k words per lane (rows lane + 64 j), and the positions of v and z in val
  constexpr int NQK = DKT / 64, VI = 2 * NQK, ZI = VI + 1, RPL = DKT / 4;
  const int C = a.C, QK = a.QK, Hv = a.Hv;
  const int npart = Hv * nblk;
  const unsigned* err = &a.ctl->error;
  // Phase B lane layout: lane 4j + p holds value column j of the slice, key rows 32p .. 32p+31.
  // The state of each head is stored transposed ([dv][dk]), so those 32 rows are contiguous.
  const int jc = lane >> 2, pr = lane & 3;
  // The slice lives in sm.sbuf (lane's chunk q at sbuf[64q + lane]); the compute waves move it
  // between HBM and LDS (state_traffic), so this wave's polls never queue behind it.
  auto fail = [&]() {
    if (lane == 0) {
      sm.abort_flag = 1;
      coherent_store_u32(&a.ctl->error, 1u);
    }
  };
  const int rep = xcd_id();
  // this XCD's copies of the broadcast buffers
  const __amdgpu_buffer_rsrc_t xrs = buf_rsrc(a.X + (size_t)rep * D, 4u * D);
  const __amdgpu_buffer_rsrc_t grs = buf_rsrc(a.G + (size_t)rep * (NCM * GSEG), 4u * NCM * GSEG);
  const bool runs_b = cw < HB && g.has_b;  // HB == 2: wave 0 the first half of the slice, wave 1 the second
  if (runs_b && cw == 0) {
    // the per-layer gates and norm weights this workgroup needs, fetched once per launch
    for (int l = lane; l < a.L; l += 64) {
      if constexpr (GT) {
        sm.gate[l][0] = *gmem(a.layers[l].a_log + g.bh);
        sm.gate[l][1] = *gmem(a.layers[l].a_bias + g.bh);
      } else {
        sm.gate[l][0] = PK ? 0.f : a.alpha[(size_t)l * Hv + g.bh];
        sm.gate[l][1] = a.beta[(size_t)l * Hv + g.bh];
      }
    }
    // sixteen loads in flight per lane before their stores (one at a time, the loop would wait a
    // memory latency per 64 values: about 30 us for the per-key decays of 30 layers)
    if constexpr (PK)
      for (int e0 = lane; e0 < a.L * DK; e0 += 64 * 16) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int e = min(e0 + 64 * u, a.L * DK - 1);
          v[u] = a.alpha[((size_t)(e / DK) * Hv + g.bh) * DK + e % DK];
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int e = e0 + 64 * u;
          if (e < a.L * DK) apk[e / DK][e % DK] = v[u];
        }
      }
    constexpr int NWC = HB * CB;  // norm weights of this workgroup's columns, per layer
    for (int e0 = lane; e0 < a.L * NWC; e0 += 64 * 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = min(e0 + 64 * u, a.L * NWC - 1);
        v[u] = *gmem(a.layers[e / NWC].norm_w + g.bcb * CB + e % NWC);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + 64 * u;
        if (e < a.L * NWC) sm.nw[e / NWC][e % NWC] = v[u];
      }
    }
  }

  // GT: this head's two gate rows (in_proj rows R + bh and R + Hv + bh), computed by the second
  // communication wave of every phase-B workgroup on the staged x while the first waits for the
  // in_proj hand-off, turned into alpha and beta and handed to phase B through LDS; their weights
  // are held one layer ahead in LDS (this wave's registers are its other work's)
  constexpr int rowbytes_in = BITS == 8 ? D : D / 2;
  const bool runs_gate = GT && cw == 1 && g.has_b;
  static_assert(NCHA <= 2, "");
  float gsc = 0.f;  // lane j < 2: the scale of gate row j
  auto load_g = [&](int l) {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the previous rows' LDS reads are done
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int8_t* wr = reinterpret_cast<const int8_t*>(a.layers[l].w_in) + (size_t)(a.R + j * Hv + g.bh) * rowbytes_in;
#pragma unroll
      for (int k = 0; k < NCHA; ++k)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const v4i*>(wr) + lane + 64 * k, &sm.gwl[j][k][0], 16, 0, 0);
    }
    gsc = lane < 2 ? *gmem(a.layers[l].s_in + a.R + lane * Hv + g.bh) : 0.f;
  };
  if (runs_gate) load_g(0);

  for (int l = 0; l < a.L; ++l) {
    const unsigned tag = base_tag + (unsigned)l;
    // Buffer base laundered once per layer: addresses derived from it are recomputed in the loop
    // (a few scalar and vector adds) instead of being held across it, which would spill.
    uint64_t* Ub = a.U;
    asm volatile("" : "+s"(Ub));
    // stage x: this wave polls a quarter of the columns (quad h of lane: columns
    // col0 + 256 h .. +3), once this workgroup's phase C of the previous layer is done
    if (cw == 0) DN_MARK(a, l, 0);
    {
      float xv[XW];
      const int col0 = cw * (D / NCM) + 4 * lane;
      bool ok = true;
      if (l == 0) {
#pragma unroll
        for (int h = 0; h < XQ; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) xv[4 * h + e] = a.x[col0 + 256 * h + e];
      } else {
        wait_counter(&sm.c_done, NCW * l, &sm.abort_flag);
        v4u q[XQ];
        unsigned w1[2] = {0u, 0u};
        ok = poll_quads<XQ, 1024, 0>(xrs, 4 * col0, 0, tag - 1, q, w1, err, a.spin_cap);
#pragma unroll
        for (int h = 0; h < XQ; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) xv[4 * h + e] = st_value(q[h][e]);
      }
      float ss = 0.f, mx = 0.f;
#pragma unroll
      for (int h = 0; h < XQ; ++h)
        *reinterpret_cast<v4f*>(sm.raw + col0 + 256 * h) = v4f{xv[4 * h], xv[4 * h + 1], xv[4 * h + 2], xv[4 * h + 3]};
#pragma unroll
      for (int i = 0; i < XW; ++i) {
        ss = fmaf(xv[i], xv[i], ss);
        mx = fmaxf(mx, fabsf(xv[i]));
      }
      ss = wave_total_f(ss);
      mx = wave_max_f(mx);
      if (lane == 0) {
        sm.stat[cw] = ss;
        sm.stat[4 + cw] = mx;
      }
      if (!__all(ok)) fail();
      if (cw == 0) DN_MARK(a, l, 1);
    }
    lds_barrier();  // (1)
    if (cw == 0) DN_MARK(a, l, 9);
    if (sm.abort_flag) break;
    split_x<BITS, D>(sm, a, tid);
    lds_barrier();  // (2)

    if (runs_gate) {
      // the head's gate rows on the staged x, into LDS for phase B; then the next layer's rows
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the rows' direct-to-LDS copies have landed
      int acc[2][3];
      v4i gw[2][NCHA];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int k = 0; k < NCHA; ++k) gw[j][k] = sm.gwl[j][k][lane];
      dot_rows<BITS, 2, NCHA>(gw, sm.xs, D, lane, acc);
      const float dot = reduce_rows<BITS, 2>(acc, sm.stat[8], lane);
      // the gate functions too run here, off the recurrence's path
      if (lane == 0) sm.gval[0] = dn_gate_alpha(gsc * dot, sm.gate[l][0], sm.gate[l][1]);
      if (lane == 1) sm.gval[1] = dn_gate_beta(gsc * dot);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the values are in LDS before the count
      asm volatile("" ::: "memory");
      if (lane == 0) bump_counter(&sm.g_ready);
      if (l + 1 < a.L) load_g(l + 1);
    }

    bool ok = true;
    if (runs_b) {
      // phase B: recurrence on the 128 x 16 state slice (HB == 2: this wave's half of the 128 x 32 one)
      const int hb = HB == 1 ? 0 : cw;
      const int vcol = g.bh * DV + (g.bcb + hb) * CB;
      // raw q and k rows lane and lane+64 of key head bg; v and z of this lane's column (HB == 2:
      // also the second half's v and z, which wave 0 hands to wave 1 through LDS)
      constexpr int NU = 2 * NQK + 2 * HB;
      float val[NU];
#pragma unroll
      for (int i = 0; i < NU; ++i) val[i] = 0.f;
      if (hb == 0) {
        const int qo = g.bg * DKT + lane;
        int off[NU];
#pragma unroll
        for (int j = 0; j < NQK; ++j) {
          off[j] = qo + 64 * j;
          off[NQK + j] = QK + qo + 64 * j;
        }
        off[VI] = 2 * QK + vcol + jc; off[ZI] = C + vcol + jc;
        if constexpr (HB == 2) {
          off[VI + 2] = 2 * QK + vcol + CB + jc;
          off[VI + 3] = C + vcol + CB + jc;
        }
        // the poll starts at once: waiting for this workgroup's own phase A first measured slower
        DN_MARK(a, l, 10);
        unsigned rounds = 0;
        ok = poll_words_at<NU>(Ub, off, tag, val, (unsigned)NU, err, a.spin_cap, &rounds);
        if (lane == 0) bump_counter(&sm.u_done);
        DN_MARK(a, l, 4);
      }
      if (__all(ok)) {
        // this wave's own LDS writes are visible to its later LDS reads (in-order LDS queue)
        if (hb == 0) {
#pragma unroll
          for (int j = 0; j < NQK; ++j) {
            sm.qk[lane + 64 * j] = val[j];
            sm.qk[DKT + lane + 64 * j] = val[NQK + j];
          }
          if constexpr (HB == 2) {
            if (pr == 0) {
              sm.vz[jc] = val[VI + 2];
              sm.vz[CB + jc] = val[VI + 3];
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): q, k, v, z are in LDS before the count
            asm volatile("" ::: "memory");
            if (lane == 0) bump_counter(&sm.v_ready);
          }
        } else if constexpr (HB == 2) {
          wait_counter(&sm.v_ready, l + 1, &sm.abort_flag);  // wave 0 has the inputs in LDS
          asm volatile("" ::: "memory");
#pragma unroll
          for (int j = 0; j < NQK; ++j) {
            val[j] = sm.qk[lane + 64 * j];
            val[NQK + j] = sm.qk[DKT + lane + 64 * j];
          }
          val[VI] = sm.vz[jc];
          val[ZI] = sm.vz[CB + jc];
        }
        DN_MARK(a, l, 11);
        float alpha = sm.gate[l][0], beta = sm.gate[l][1];
        if constexpr (GT) {
          wait_counter(&sm.g_ready, l + 1, &sm.abort_flag);  // this head's gate values are in LDS
          asm volatile("" ::: "memory");
          alpha = sm.gval[0];
          beta = sm.gval[1];
        }
        const v4f* Q4 = reinterpret_cast<const v4f*>(sm.qk + RPL * pr);
        const v4f* K4 = reinterpret_cast<const v4f*>(sm.qk + DKT + RPL * pr);
        const v4f* A4 = reinterpret_cast<const v4f*>(&apk[PK ? l : 0][RPL * pr]);
        float sv[RPL];
        float kvp = 0.f, qvp = 0.f, kqp = 0.f;
        wait_counter(&sm.s_ready, NCW * (l + 1), &sm.abort_flag);  // the slice has landed in LDS
        // the sums run over the raw q and k; the 1/norm factors multiply the finished sums (and the
        // delta), so the fp64 norm reductions below can overlap the state arithmetic. The readout
        // over the updated state, (S' )^T q = (decayed S)^T q + delta (k . q), takes its sums in the
        // same pass, so it is published before the update of the slice.
#pragma unroll
        for (int q = 0; q < RPL / 4; ++q) {
          const v4f kk = K4[q], qq = Q4[q], st = sm.sbuf[hb][64 * q + lane];
          v4f av = {alpha, alpha, alpha, alpha};  // decay of rows 32 pr + 4 q ..
          if constexpr (PK) av = A4[q];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sv[4 * q + e] = av[e] * st[e];  // decay
            kvp = fmaf(sv[4 * q + e], kk[e], kvp);
            qvp = fmaf(sv[4 * q + e], qq[e], qvp);
            kqp = fmaf(kk[e], qq[e], kqp);
          }
        }
        // L2 norms in double, eps inside the sqrt (independent of the loop above, so the two overlap)
        double sq0 = 0.0, sk0 = 0.0;
#pragma unroll
        for (int j = 0; j < NQK; ++j) {
          sq0 += (double)val[j] * val[j];
          sk0 += (double)val[NQK + j] * val[NQK + j];
        }
        const double sq = wave_total_d(sq0);
        const double sk = wave_total_d(sk0);
        const float qn = (float)((double)a.q_scale / sqrt(sq + (double)a.eps_l2));
        const float kn = (float)(1.0 / sqrt(sk + (double)a.eps_l2));
        const float kv = kn * quad_sum(kvp);  // (decayed S)^T k^ of column jc
        const float dk = beta * (val[VI] - kv) * kn;  // delta times 1/|k|
        DN_MARK(a, l, 13);
        const float o = qn * fmaf(dk, quad_sum(kqp), quad_sum(qvp));
        const float gt = sm.nw[l][hb * CB + jc] * o * silu(val[ZI]);
        const float osq = wave_total_f(pr == 0 ? o * o : 0.f);
        DN_MARK(a, l, 15);
        // G buffer: NCM segments of [V/NCM gated columns | partials of the same heads]
        const int gc = vcol + jc, gw = gc / (V / NCM);
        const int pw = g.bh / (Hv / NCM);
        // the four lanes of column jc hold the same value: lane 4jc+p writes replicas 2p and 2p+1;
        // lanes 0..7 write one replica each of the partial sum
        {
          const size_t off = (size_t)gw * GSEG + (gc - gw * (V / NCM));
          const int r0 = 2 * pr;
          const int unit = HB * wg + hb;  // = nblk * bh + this half's column block
          if constexpr (HB == 2) {
            const int poff = pw * GSEG + V / NCM + (unit - pw * (npart / NCM));  // (through a buffer resource: no 64-bit address kept per lane)
            const __amdgpu_buffer_rsrc_t gall = buf_rsrc(a.G, 4u * NREP * NCM * GSEG);
            st_store_rs(gall, 4 * (r0 * (NCM * GSEG) + (int)off), gt, tag);
            st_store_rs(gall, 4 * ((r0 + 1) * (NCM * GSEG) + (int)off), gt, tag);
            if (lane < NREP) st_store_rs(gall, 4 * (lane * (NCM * GSEG) + poff), osq, tag);
          } else {
            st_store(a.G + (size_t)r0 * (NCM * GSEG) + off, gt, tag);
            st_store(a.G + (size_t)(r0 + 1) * (NCM * GSEG) + off, gt, tag);
            if (lane < NREP)
              st_store(a.G + (size_t)lane * (NCM * GSEG) + pw * GSEG + V / NCM + (unit - pw * (npart / NCM)), osq, tag);
          }
        }
        // the delta rule write, after the readout is out; the slice is parked in LDS and written
        // back while phase C runs
#pragma unroll
        for (int q = 0; q < RPL / 4; ++q) {
          const v4f kk = K4[q];
#pragma unroll
          for (int e = 0; e < 4; ++e) sv[4 * q + e] = fmaf(kk[e], dk, sv[4 * q + e]);
          sm.sbuf[hb][q * 64 + lane] = v4f{sv[4 * q], sv[4 * q + 1], sv[4 * q + 2], sv[4 * q + 3]};
        }
        DN_MARK(a, l, 14);
        DN_MARK(a, l, 5);
      }
      if (lane == 0) bump_counter(&sm.b_done);
    } else if (cw == 0) {
      wait_counter(&sm.a_done, NCW * (l + 1), &sm.abort_flag);
      if (lane == 0) {
        bump_counter(&sm.u_done);
#pragma unroll
        for (int h = 0; h < HB; ++h) bump_counter(&sm.b_done);
      }
    }
    if (__all(ok)) {
      // stage the gated readout: value columns [cw*V/NCM, (cw+1)*V/NCM) and the partials of those
      // heads, which follow them in this wave's segment of the buffer
      wait_counter(&sm.b_done, HB * (l + 1), &sm.abort_flag);
      float gv[GW + HB];
      const int pn = npart / NCM, pbase = cw * pn;
      if (cw == 0) DN_MARK(a, l, 12);
      {
        // quad h of lane: columns cw V/4 + 256 h + 4 lane .. +3; then the partial of lane (< pn)
        // the partials of this quarter's heads: HB consecutive ones per lane (lanes < pn / HB)
        v4u q[GQ];
        unsigned w1[2] = {0u, 0u};
        const int w0 = cw * GSEG + 4 * lane;
        if (HB * lane < pn)
          ok = poll_quads<GQ, 1024, HB>(grs, 4 * w0, 4 * (cw * GSEG + V / NCM + HB * lane), tag, q, w1, err, a.spin_cap);
        else
          ok = poll_quads<GQ, 1024, 0>(grs, 4 * w0, 0, tag, q, w1, err, a.spin_cap);
#pragma unroll
        for (int h = 0; h < GQ; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) gv[4 * h + e] = st_value(q[h][e]);
#pragma unroll
        for (int h = 0; h < HB; ++h) gv[GW + h] = HB * lane < pn ? st_value(w1[h]) : 0.f;
      }
      if (cw == 0) DN_MARK(a, l, 6);
      // per-head sums of the partials: head h's nblk partials sit in nblk / HB consecutive lanes
      {
        static_assert(nblk == 8 || (nblk == 16 && HB == 1), "");
        if constexpr (HB == 1) {
          float sp = oct_sum(gv[GW]);
          if constexpr (nblk == 16) sp += __int_as_float(dpp_i<0x140>(__float_as_int(sp)));  // mirrored row of 16
          if ((lane % nblk) == 0 && lane < pn) sm.inv[(pbase + lane) / nblk] = rsqrtf(sp / (float)DV + a.eps_rms);
        } else {
          const float sp = quad_sum(gv[GW] + gv[GW + 1]);
          if ((lane % 4) == 0 && 2 * lane < pn) sm.inv[(pbase + 2 * lane) / nblk] = rsqrtf(sp / (float)DV + a.eps_rms);
        }
      }
      // y = g / rms(head), staged for phase C, and the sum of this quarter of y
      float sy = 0.f;
      const int gcol0 = cw * (V / NCM) + 4 * lane;
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        const int c = gcol0 + 256 * h;  // the four columns of a quad belong to one head
        const float iv = sm.inv[c / DV];
        const v4f y = v4f{gv[4 * h], gv[4 * h + 1], gv[4 * h + 2], gv[4 * h + 3]} * iv;
        *reinterpret_cast<v4f*>(sm.yf + ypos<BITS>(c)) = y;
        sy += (y[0] + y[1]) + (y[2] + y[3]);
      }
      sy = wave_total_f(sy);
      if (lane == 0) sm.stat[9 + cw] = sy;
    }
    if (!__all(ok)) fail();
    if (cw == 0) DN_MARK(a, l, 29);
    lds_barrier();  // (3)
    if (sm.abort_flag) break;
  }
}

template <int BITS, int NCHA, int NCHC, int RA, int RC, bool PK, bool GT, int HB, int DKT = DK>
__global__ __launch_bounds__(NTHR) void k_persist(const PersistArgs a) {
  constexpr int COLS_PER_CHUNK = BITS == 8 ? 1024 : 2048;
  constexpr int D = COLS_PER_CHUNK * NCHA;
  constexpr int nblk = DKT / CB;  // column blocks per value head (dv = dk)
  __shared__ SmemT<HB, DKT> sm;
  __shared__ float apk[PK ? PK_MAXL : 1][DK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NWG = gridDim.x, wg = blockIdx.x;
  const unsigned base_tag = coherent_load_u32(&a.ctl->epoch);
  // A launch after one that abandoned its token does nothing (the error flag is sticky until the
  // host restarts the handle), so the current buffers keep the state before the abandoned token.
  const bool skip = coherent_load_u32(&a.ctl->error) != 0;
  const unsigned par = coherent_load_u32(&a.ctl->parity) & 1u;

  Geo g;
  const int a_per_wg = (a.R + NWG - 1) / NWG;
  g.a_per_wg = a_per_wg;
  const int a_per_wave = (a_per_wg + NCW - 1) / NCW;
  g.a_row0 = wg * a_per_wg + wave * a_per_wave;
  g.a_row_end = min(min(wg * a_per_wg + a_per_wg, a.R), g.a_row0 + a_per_wave);
  const int c_per_wg = (D + NWG - 1) / NWG;
  const int c_per_wave = (c_per_wg + NCW - 1) / NCW;
  g.c_row0 = wg * c_per_wg + wave * c_per_wave;
  g.c_row_end = min(min(wg * c_per_wg + c_per_wg, D), g.c_row0 + c_per_wave);
  // phase-B workgroups: nblk / HB per value head, each HB column blocks of it (bcb the first)
  constexpr int WPH = nblk / HB;
  g.has_b = wg < a.Hv * WPH;
  g.bh = g.has_b ? wg / WPH : 0;
  g.bcb = g.has_b ? HB * (wg % WPH) : 0;
  g.bg = g.bh / (a.Hv / a.Hk);

  if (tid == 0) {
    sm.abort_flag = 0;
    sm.a_done = sm.b_done = sm.c_done = sm.u_done = sm.s_ready = sm.g_ready = 0;
    if constexpr (HB == 2) sm.v_ready = 0;
  }
#ifdef DN_PHASE_TIMERS
  for (int e = tid; e < TS_MAXL * 32; e += NTHR) g_ts[e / 32][e % 32] = 0;
#endif
  __syncthreads();
  // The two roles run separate loops with the same sequence of three workgroup barriers per
  // layer, so each role's registers are its own. Reads come from the current buffers (par), writes
  // go to the other ones.
  if (!skip) {
    if (wave < NCW)
      compute_role<BITS, NCHA, NCHC, RA, RC, PK, GT, HB, DKT>(sm, a, g, base_tag, a.S[par], a.S[par ^ 1u], a.ring[par],
                                                     a.ring[par ^ 1u], tid, lane);
    else
      comm_role<BITS, NCHA, NCHC, PK, GT, HB, DKT>(sm, apk, a, g, base_tag, tid, lane, wave - NCW, wg);
  }

#ifdef DN_PHASE_TIMERS
  __syncthreads();
  for (int e = tid; e < min(a.L, TS_MAXL) * 32; e += NTHR)
    a.timers[((size_t)blockIdx.x * a.L + e / 32) * 32 + e % 32] = g_ts[e / 32][e % 32];
#endif
  // The last workgroup to finish advances the tag base for the next launch and, if no workgroup
  // failed, makes the written buffers current; every workgroup's stores have completed before its
  // count (the barrier's fence waits for them).
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(&a.ctl->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == (unsigned)NWG - 1) {
      const unsigned err = coherent_load_u32(&a.ctl->error);
      coherent_store_u32(&a.ctl->done, 0u);
      coherent_store_u32(&a.ctl->epoch, base_tag + (unsigned)a.L);
      if (!err) coherent_store_u32(&a.ctl->parity, par ^ 1u);
      // publish this launch's error flag to the host without a copy on the stream
      __hip_atomic_store(a.err_host, err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
}

template <typename F>
hipError_t launch_one(F kern, const PersistArgs& a, int nwg, bool coop, hipStream_t st) {
  if (coop) {
    // the runtime starts the grid only when every workgroup can be resident at once
    void* args[] = {const_cast<PersistArgs*>(&a)};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kern), dim3(nwg), dim3(NTHR), args, 0, st);
  }
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(NTHR), 0, st, a);
  return hipGetLastError();
}

// 48 value heads of 128 over d_model 2048 (8-bit): 64 in_proj rows per workgroup (8 per compute
// wave), the state in 128 x 32 slices (two phase-B waves), caller-given scalar decays
hipError_t go_hb2(const PersistArgs& a, int nwg, bool coop, hipStream_t st) {
  return launch_one(k_persist<8, 2, 6, 8, 1, false, false, 2>, a, nwg, coop, st);
}
// heads of 256 (dk = dv = 256) over d_model 2048 (8-bit), value width 4096: 256 x 16 state slices,
// 64 key rows per lane of the phase-B wave, caller-given scalar decays
hipError_t go_dk256(const PersistArgs& a, int nwg, bool coop, hipStream_t st) {
  return launch_one(k_persist<8, 2, 4, 6, 1, false, false, 1, 256>, a, nwg, coop, st);
}

template <int BITS, int NCHA, int NCHC>
hipError_t go(const PersistArgs& a, int nwg, bool coop, hipStream_t st) {
  if (a.alpha_per_key) return launch_one(k_persist<BITS, NCHA, NCHC, 6, 1, true, false, 1>, a, nwg, coop, st);
  if (a.gates) return launch_one(k_persist<BITS, NCHA, NCHC, 6, 1, false, true, 1>, a, nwg, coop, st);
  return launch_one(k_persist<BITS, NCHA, NCHC, 6, 1, false, false, 1>, a, nwg, coop, st);
}

template <int BITS, int NCHA, int NCHC>
hipError_t occ(int* blocks, bool pk, bool gt) {
  if (pk) return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, k_persist<BITS, NCHA, NCHC, 6, 1, true, false, 1>, NTHR, 0);
  if (gt) return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, k_persist<BITS, NCHA, NCHC, 6, 1, false, true, 1>, NTHR, 0);
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, k_persist<BITS, NCHA, NCHC, 6, 1, false, false, 1>, NTHR, 0);
}

}  // namespace

// Chunk counts (16-byte chunks per lane) of an in_proj and out_proj row, or 0 if unsupported.
static int chunks(int cols, int bits) {
  const int bytes = bits == 8 ? cols : cols / 2;
  if (bytes % 1024) return 0;
  return bytes / 1024;
}

// The two-wave instantiation's shape: 8-bit weights, d_model 2048, value width 6144 (48 heads of 128),
// caller-given scalar decays, at most 64 layers, 8 in_proj rows per compute wave.
static bool hb2_shape(const PersistShape& s, int nwg) {
  if (s.batch != 1 || s.dk != DK || s.dv != 128 || s.K < 1 || s.K > 4 || s.bits != 8) return false;
  if (s.alpha_per_key || s.gates || s.L > SmemT<2>::LMAX) return false;
  if (chunks(s.D, s.bits) != 2 || chunks(s.V, s.bits) != 6 || (s.Hv % NCM) || s.Hv > 64) return false;
  if (s.Hv * (s.dv / CB) / 2 > nwg) return false;
  const int a_per_wg = (s.R + nwg - 1) / nwg, c_per_wg = (s.D + nwg - 1) / nwg;
  return (a_per_wg + NCW - 1) / NCW <= 8 && (c_per_wg + NCW - 1) / NCW <= 1;
}

// The heads-of-256 instantiation's shape: 8-bit weights, d_model 2048, value width 4096, dk = dv = 256,
// caller-given scalar decays, one 256 x 16 slice per workgroup.
static bool dk256_shape(const PersistShape& s, int nwg) {
  if (s.batch != 1 || s.dk != 256 || s.dv != 256 || s.K < 1 || s.K > 4 || s.bits != 8) return false;
  if (s.alpha_per_key || s.gates) return false;
  if (chunks(s.D, s.bits) != 2 || chunks(s.V, s.bits) != 4 || (s.Hv % NCM) || s.Hv * (s.dv / CB) > nwg) return false;
  const int a_per_wg = (s.R + nwg - 1) / nwg, c_per_wg = (s.D + nwg - 1) / nwg;
  return (a_per_wg + NCW - 1) / NCW <= 6 && (c_per_wg + NCW - 1) / NCW <= 1;
}

bool persist_supported(const PersistShape& s, int nwg) {
  if (hb2_shape(s, nwg) || dk256_shape(s, nwg)) return true;
  if (s.batch != 1 || s.dk != DK || s.dv != 128 || s.K < 1 || s.K > 4) return false;
  if (s.alpha_per_key && s.L > PK_MAXL) return false;
  if (s.alpha_per_key && s.gates) return false;
  if (s.gates && 2 * s.Hv > nwg) return false;
  const int na = chunks(s.D, s.bits), nc = chunks(s.V, s.bits);
  const bool inst = s.bits == 8 ? ((na == 2 && nc == 4) || (na == 1 && nc == 1))
                                : ((na == 1 && nc == 2) || (na == 1 && nc == 1));
  if (!inst) return false;
  if (s.D > 4096 || s.V > 4096 || s.Hv > 32 || (s.Hv % NCM)) return false;
  if (s.Hv * (s.dv / CB) > nwg) return false;
  const int a_per_wg = (s.R + nwg - 1) / nwg, c_per_wg = (s.D + nwg - 1) / nwg;
  if ((a_per_wg + NCW - 1) / NCW > 6 || (c_per_wg + NCW - 1) / NCW > 1) return false;
  return true;
}

hipError_t persist_occupancy(const PersistShape& s, int* blocks_per_cu) {
  const int na = chunks(s.D, s.bits), nc = chunks(s.V, s.bits);
  const bool pk = s.alpha_per_key != 0, gt = s.gates != 0;
  if (s.bits == 8 && na == 2 && nc == 6)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, k_persist<8, 2, 6, 8, 1, false, false, 2>, NTHR, 0);
  if (s.dk == 256)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, k_persist<8, 2, 4, 6, 1, false, false, 1, 256>, NTHR, 0);
  if (s.bits == 8) return na == 2 ? occ<8, 2, 4>(blocks_per_cu, pk, gt) : occ<8, 1, 1>(blocks_per_cu, pk, gt);
  return nc == 2 ? occ<4, 1, 2>(blocks_per_cu, pk, gt) : occ<4, 1, 1>(blocks_per_cu, pk, gt);
}

hipError_t launch_persist(const PersistArgs& a, const PersistShape& s, int nwg, bool coop, hipStream_t st) {
  const int na = chunks(s.D, s.bits), nc = chunks(s.V, s.bits);
  if (s.bits == 8 && na == 2 && nc == 6) return go_hb2(a, nwg, coop, st);
  if (s.dk == 256) return go_dk256(a, nwg, coop, st);
  if (s.bits == 8) return na == 2 ? go<8, 2, 4>(a, nwg, coop, st) : go<8, 1, 1>(a, nwg, coop, st);
  return nc == 2 ? go<4, 1, 2>(a, nwg, coop, st) : go<4, 1, 1>(a, nwg, coop, st);
}


// Canonical state [L][Hv][dk][dv] <-> the whole-stack kernel's layout [L][Hv][dv][dk] (each head transposed).
__global__ void k_state_tile(const float* __restrict__ src, float* __restrict__ dst, int L, int Hv, int dk, int dv,
                             int to_tiled) {
  const size_t n = (size_t)L * Hv * dk * dv;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
    const int j = (int)(e % dv);
    size_t t = e / dv;
    const int i = (int)(t % dk);
    t /= dk;  // l * Hv + h
    const size_t tiled = (t * dv + j) * dk + i;  // each head stored transposed, [dv][dk]
    if (to_tiled) dst[tiled] = src[e];
    else dst[e] = src[tiled];
  }
}

hipError_t launch_state_tile(const float* src, float* dst, int L, int Hv, int dk, int dv, bool to_tiled,
                             hipStream_t st) {
  hipLaunchKernelGGL(k_state_tile, dim3(1024), dim3(256), 0, st, src, dst, L, Hv, dk, dv, to_tiled ? 1 : 0);
  return hipGetLastError();
}

}  // namespace dn
