// pararnn.hip -- gfx950 (MI355X) kernels and C ABI of libpararnn.so.
//
// The ParaRNN hot path (pararnn-torch README on PyPI, section "Method"; ParaRNN
// abstract on the HF paper list): the trajectory H of a nonlinear recurrence
// h_t = f(h_{t-1}, x_t) is the unknown of F(H)_t = h_t - f(h_{t-1}, x_t) = 0;
// Newton iterations solve it, and each iteration's linearised system is a
// first-order linear recurrence solved by a parallel prefix scan along T.  The
// backward pass is the adjoint: a reverse scan with transposed Jacobians.
//
// Design (MI355X first):
//  * Channels (b, d) are independent for diagonal cells.  A workgroup tile is
//    TW = 64*V consecutive channels (lane = V channels, loads of 4..16 bytes
//    per lane, a wave reads one contiguous row) by CT = NW*L time steps (wave
//    w owns steps [w*L, (w+1)*L) of the chunk, each lane walks its L steps
//    serially in registers).  The diagonal cells use no MFMA (no step is a
//    dense contraction): a kernel that runs one iteration per launch is bound
//    by HBM bandwidth, the fused pass that runs several (k_fused) by vector
//    ALU issue.  The head-wise block GRU (head_gru_dev.inc) composes its dense
//    Jacobian blocks on MFMA.
//  * One kernel per scan / Newton iteration / VJP (the fused pass: several
//    iterations per launch, trajectory kept on chip).  Each tile (1) produces its
//    affine scan elements in registers (loaded, or computed from the cell's
//    residual and Jacobian), (2) reduces them per lane and across waves
//    through LDS, (3) obtains the state entering its chunk by a decoupled
//    look-back over the tiles before it in scan order, (4) re-walks its
//    elements from that state and writes the result.  Inputs are read once.
//  * The look-back exchanges 64-bit words (32-bit launch tag | fp32 value):
//    a word is valid when its tag matches the launch, so no flags, fences or
//    cache maintenance are needed; words are relaxed agent-scope atomics.
//    Tiles take their position from an atomic ticket, so every tile a tile
//    waits on is already running (forward progress without co-residency).
//  * Newton iterations update the trajectory in place; the one value a tile
//    needs from its predecessor's chunk (h_{t0-1}) travels as a look-back word.
//
// Compile with -Xclang -target-feature -Xclang -packed-fp32-ops (no packed
// fp32 instructions are generated).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstddef>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "pararnn.h"
#include "pararnn_debug.h"

#define DEV __device__ __forceinline__

namespace pr {

constexpr int WAVE = 64;
enum { CELL_LINEAR = 0, CELL_GRU = 1, CELL_LSTM = 2, CELL_SLSTM = 3, CELL_HEAD_GRU = 4 };
enum { DT_F32 = 0, DT_BF16 = 1 };

// ------------------------------------------------------------------------------------------------
// device math: exp and reciprocal from the hardware transcendental unit (v_exp_f32 is 2^x,
// v_rcp_f32 is 1/x, each about 1 ulp); sigmoid and tanh from their definitions.
// ------------------------------------------------------------------------------------------------
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
DEV float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
DEV float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
DEV float sigmoid(float x) { return hw_rcp(1.0f + hw_exp2(-kLog2e * x)); }
// tanh(x) = 1 - 2 / (1 + e^{2x})
DEV float tanh_(float x) { return fmaf(-2.0f, hw_rcp(1.0f + hw_exp2(2.0f * kLog2e * x)), 1.0f); }
// maximum that lets a NaN win, so a NaN residual is never hidden
DEV float nanmax(float m, float x) { return (x > m || x != x) ? x : m; }

// ------------------------------------------------------------------------------------------------
// vector loads / stores of V consecutive channels.  Streaming data (read or written once per pass) is
// stored non-temporally (PR_NT_STORE); fp32 planes are loaded non-temporally too (PR_NT_F32: a wave's row of
// them fills whole cache lines), bf16 planes through the cache (PR_NT_BF16 = 0: a time slice's row is half a
// line, whose other half the neighbouring channel tile reads soon after).
// ------------------------------------------------------------------------------------------------
#ifndef PR_NT_F32
#define PR_NT_F32 1
#endif
#ifndef PR_NT_BF16
#define PR_NT_BF16 0
#endif
#ifndef PR_NT_STORE
#define PR_NT_STORE 1
#endif
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <bool NT, typename T>
DEV T ld_stream(const T* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <typename T>
DEV void st_stream(T* p, T v) {
  if constexpr (PR_NT_STORE) __builtin_nontemporal_store(v, p);
  else *p = v;
}

template <int V, int DT>
DEV void ldv(const void* base, int64_t idx, float (&o)[V]) {
  if constexpr (DT == DT_F32) {
    constexpr bool NT = PR_NT_F32;
    const float* p = static_cast<const float*>(base) + idx;
    if constexpr (V == 1) {
      o[0] = ld_stream<NT>(p);
    } else if constexpr (V == 2) {
      const f32x2 t = ld_stream<NT>(reinterpret_cast<const f32x2*>(p));
      o[0] = t.x; o[1] = t.y;
    } else {
      const f32x4 t = ld_stream<NT>(reinterpret_cast<const f32x4*>(p));
      o[0] = t.x; o[1] = t.y; o[2] = t.z; o[3] = t.w;
    }
  } else {
    const uint16_t* p = static_cast<const uint16_t*>(base) + idx;
    if constexpr (V == 1) {
      o[0] = __uint_as_float(static_cast<uint32_t>(ld_stream<PR_NT_BF16>(p)) << 16);
    } else if constexpr (V == 2) {
      const uint32_t t = ld_stream<PR_NT_BF16>(reinterpret_cast<const uint32_t*>(p));
      o[0] = __uint_as_float(t << 16); o[1] = __uint_as_float(t & 0xffff0000u);
    } else {
      const u32x2 t = ld_stream<PR_NT_BF16>(reinterpret_cast<const u32x2*>(p));
      o[0] = __uint_as_float(t.x << 16); o[1] = __uint_as_float(t.x & 0xffff0000u);
      o[2] = __uint_as_float(t.y << 16); o[3] = __uint_as_float(t.y & 0xffff0000u);
    }
  }
}

// small per-channel parameter vectors (re-read by every tile): plain cached loads
template <int V>
DEV void ldv_param(const float* base, int64_t idx, float (&o)[V]) {
  const float* p = base + idx;
#pragma unroll
  for (int v = 0; v < V; ++v) o[v] = p[v];
}

template <int V>
DEV void stv(float* p, const float (&x)[V]) {
  if constexpr (V == 1) {
    st_stream(p, x[0]);
  } else if constexpr (V == 2) {
    st_stream(reinterpret_cast<f32x2*>(p), f32x2{x[0], x[1]});
  } else {
    st_stream(reinterpret_cast<f32x4*>(p), f32x4{x[0], x[1], x[2], x[3]});
  }
}

// the same loads and stores addressed as a uniform base element plus the lane's 32-bit offset, so
// that each one is a scalar base register and one vector offset (no per-load 64-bit vector adds)
template <int V, int DT>
DEV void ldv_u(const void* plane, int64_t ubase, uint32_t loff, float (&o)[V]) {
  constexpr int ESZ = DT == DT_F32 ? 4 : 2;
  const char* p = static_cast<const char*>(plane) + ubase * ESZ + static_cast<uint64_t>(loff * ESZ);
  ldv<V, DT>(p, 0, o);
}
// raw buffer view of one plane from a uniform base address: a load is (descriptor, 32-bit lane
// byte offset, 32-bit uniform byte offset) with no vector address arithmetic at all.  Word 3 is
// the raw-buffer format of the gfx9 family; the 4 GiB record count disables range checking
// within the window (callers keep every offset inside the plane).
#ifndef PR_FAST_S2
#define PR_FAST_S2 1
#endif
typedef __amdgpu_buffer_rsrc_t Rsrc;
DEV Rsrc rsrc_at(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), -1, 0x00020000);
}
template <int V, int DT>
DEV void ldv_buf(Rsrc r, uint32_t voff, uint32_t soff, float (&o)[V]) {
  constexpr int AUX = (DT == DT_F32 ? PR_NT_F32 : PR_NT_BF16) ? 2 : 0;   // cache policy 2: non-temporal
  if constexpr (DT == DT_F32) {
    if constexpr (V == 1) {
      o[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, AUX));
    } else if constexpr (V == 2) {
      const auto t = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, AUX);
      o[0] = __uint_as_float(t[0]); o[1] = __uint_as_float(t[1]);
    } else {
      const auto t = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX);
      o[0] = __uint_as_float(t[0]); o[1] = __uint_as_float(t[1]);
      o[2] = __uint_as_float(t[2]); o[3] = __uint_as_float(t[3]);
    }
  } else {
    if constexpr (V == 1) {
      o[0] = __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, AUX)) << 16);
    } else if constexpr (V == 2) {
      const uint32_t t = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, AUX);
      o[0] = __uint_as_float(t << 16); o[1] = __uint_as_float(t & 0xffff0000u);
    } else {
      const auto t = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, AUX);
      o[0] = __uint_as_float(t[0] << 16); o[1] = __uint_as_float(t[0] & 0xffff0000u);
      o[2] = __uint_as_float(t[1] << 16); o[3] = __uint_as_float(t[1] & 0xffff0000u);
    }
  }
}

template <int V>
DEV void stv_u(float* plane, int64_t ubase, uint32_t loff, const float (&x)[V]) {
  char* p = reinterpret_cast<char*>(plane + ubase) + static_cast<uint64_t>(loff * 4u);
  stv<V>(reinterpret_cast<float*>(p), x);
}

// ------------------------------------------------------------------------------------------------
// affine maps x -> A x + b on the S-dimensional state (Blelloch's first-order-recurrence
// operator).  compose(later, earlier) = later o earlier; associative, not commutative.
// ------------------------------------------------------------------------------------------------
template <int S>
struct Aff {
  float A[S * S];
  float b[S];
};

template <int S>
DEV Aff<S> aff_id() {
  Aff<S> m;
#pragma unroll
  for (int i = 0; i < S; ++i) {
#pragma unroll
    for (int j = 0; j < S; ++j) m.A[i * S + j] = (i == j) ? 1.0f : 0.0f;
    m.b[i] = 0.0f;
  }
  return m;
}

template <int S>
DEV Aff<S> compose(const Aff<S>& lat, const Aff<S>& ear) {
  Aff<S> r;
#pragma unroll
  for (int i = 0; i < S; ++i) {
#pragma unroll
    for (int j = 0; j < S; ++j) {
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k < S; ++k) acc = fmaf(lat.A[i * S + k], ear.A[k * S + j], acc);
      r.A[i * S + j] = acc;
    }
    float acc = lat.b[i];
#pragma unroll
    for (int k = 0; k < S; ++k) acc = fmaf(lat.A[i * S + k], ear.b[k], acc);
    r.b[i] = acc;
  }
  return r;
}

template <int S>
DEV void apply(const Aff<S>& m, float (&x)[S]) {
  float y[S];
#pragma unroll
  for (int i = 0; i < S; ++i) {
    float acc = m.b[i];
#pragma unroll
    for (int k = 0; k < S; ++k) acc = fmaf(m.A[i * S + k], x[k], acc);
    y[i] = acc;
  }
#pragma unroll
  for (int i = 0; i < S; ++i) x[i] = y[i];
}

// compose and apply for an element whose matrix is known to be zero outside MASK (bit i*S + k set where
// A[i][k] may be nonzero): the skipped terms are exact zeros, so the result equals compose / apply for finite
// values, with fewer multiply-adds (the sLSTM's 4x4 Jacobian has four structural zeros and a sparse row)
template <int S, uint32_t MASK>
DEV Aff<S> compose_masked(const Aff<S>& lat, const Aff<S>& ear) {
  Aff<S> r;
#pragma unroll
  for (int i = 0; i < S; ++i) {
#pragma unroll
    for (int j = 0; j < S; ++j) {
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k < S; ++k)
        if ((MASK >> (i * S + k)) & 1u) acc = fmaf(lat.A[i * S + k], ear.A[k * S + j], acc);
      r.A[i * S + j] = acc;
    }
    float acc = lat.b[i];
#pragma unroll
    for (int k = 0; k < S; ++k)
      if ((MASK >> (i * S + k)) & 1u) acc = fmaf(lat.A[i * S + k], ear.b[k], acc);
    r.b[i] = acc;
  }
  return r;
}
template <int S, uint32_t MASK>
DEV void apply_masked(const Aff<S>& m, float (&x)[S]) {
  float y[S];
#pragma unroll
  for (int i = 0; i < S; ++i) {
    float acc = m.b[i];
#pragma unroll
    for (int k = 0; k < S; ++k)
      if ((MASK >> (i * S + k)) & 1u) acc = fmaf(m.A[i * S + k], x[k], acc);
    y[i] = acc;
  }
#pragma unroll
  for (int i = 0; i < S; ++i) x[i] = y[i];
}
template <int S>
constexpr uint32_t kFullMask = (S * S >= 32) ? 0xFFFFFFFFu : ((1u << (S * S)) - 1u);
// the sLSTM Jacobian (state c, n, m, h): c' and n' do not depend on n and c respectively, m' not on c or n
constexpr uint32_t kSlstmJMask = 0xFCEDu;
// its transpose (the VJP's elements)
constexpr uint32_t kSlstmJtMask = 0xFFA9u;

template <int S>
DEV float aff_get(const Aff<S>& m, int k) { return k < S * S ? m.A[k] : m.b[k - S * S]; }
template <int S>
DEV void aff_set(Aff<S>& m, int k, float v) {
  if (k < S * S) m.A[k] = v; else m.b[k - S * S] = v;
}

// ------------------------------------------------------------------------------------------------
// look-back words: (tag << 32) | float bits, relaxed agent-scope atomics.
// Layout: word (p, chain, slot, q) at ((p * n_chains + chain) * n_slots + slot) * TW + q, where p is
// the tile's position in scan order and q its channel within the tile.
// ------------------------------------------------------------------------------------------------
DEV uint64_t ld_word(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV void st_word(uint64_t* p, uint32_t tag, float v) {
  const uint64_t w = (static_cast<uint64_t>(tag) << 32) | __float_as_uint(v);
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV bool word_ok(uint64_t w, uint32_t tag) { return static_cast<uint32_t>(w >> 32) == tag; }
DEV float word_val(uint64_t w) { return __uint_as_float(static_cast<uint32_t>(w)); }

struct Common {
  uint64_t* lb;         // look-back words
  const uint32_t* seg;  // packed sequences: bit t set where a sequence other than the first begins
  uint32_t* ticket;     // tile ticket counter of this launch (zeroed before the launch)
  uint32_t tag;         // nonzero tag of this launch
  int32_t n_chains;     // channel tiles
  int64_t n_chunks;     // time chunks
  int64_t T, D, C, N;   // time steps, channels per row, B*D channels, B*T*D elements
  int32_t off32;        // every lane's offset from its wave's base element fits 32 bits (in bytes
                        // of fp32): full tiles address memory as uniform base + 32-bit offset
};

// Packed sequences: 32 mask bits starting at step t0 (bit i <-> step t0 + i).  The mask has
// (T >> 5) + 2 words and no bit at or past T, so the two words read are in bounds for any
// t0 <= T; lanes whose steps lie past T read some in-bounds word and mask those steps anyway.
DEV uint32_t seg_bits(const uint32_t* seg, int64_t t0, int64_t T) {
  const int64_t tc = t0 < T ? t0 : T;
  const int64_t w = tc >> 5;
  const uint64_t win = (static_cast<uint64_t>(seg[w + 1]) << 32) | seg[w];
  return static_cast<uint32_t>(win >> (tc & 31));
}

// A tile is TW channels x CT steps.  A wave's 64 lanes form TS time slices of 64/TS lanes; lane
// (slice s, position j) owns channels [j*V, j*V+V) of the tile and L consecutive steps; the NW*TS
// segments of L steps are stacked in time: wave w, slice s -> segment w*TS + s.
struct Tile {
  int64_t p, chunk, t_lo, ch0, b, d0;
  int64_t wbase;     // uniform over the wave: element (row, step, channel) of the wave's first lane
  uint32_t loff;     // this lane's element offset from wbase (valid when Common::off32)
  int chain, wave, lane, slice, qlane;
  int nvalid;        // steps of this lane inside [0, T); the same for every lane of a slice
  bool active;       // the lane's channels exist
  bool first_seg;    // this lane holds the tile's first segment in time (wave 0, slice 0)
  bool last_seg;     // ... the tile's last segment in time
};

// row of step t clamped into [0, T): loads use clamped addresses and masked steps are replaced by
// identity elements afterwards, so the load phase has no branches and every load is in flight at once
DEV int64_t clamp_t(int64_t t, int64_t T) { return t < 0 ? 0 : (t >= T ? T - 1 : t); }

template <int S, int TW, int NSLOT>
DEV uint64_t* word_at(const Common& c, int64_t p, int chain, int slot, int q) {
  return c.lb + ((p * c.n_chains + chain) * NSLOT + slot) * static_cast<int64_t>(TW) + q;
}

// Debug builds (-DPR_LB_STRESS=1) pause the tiles that publish look-back words for a pseudo-random time,
// different for every launch, tile and call site, so that the words appear in a scrambled order and walks
// reach far back; the library built so must give the same bits as the plain one.  Every pause is bounded.
#ifndef PR_LB_STRESS
#define PR_LB_STRESS 0
#endif
#if PR_LB_STRESS
__device__ uint32_t g_lb_max_depth;   // deepest walk seen: aggregates applied to an inclusive word (0 or 1)
#endif
DEV void stress_pause(const Common& c, int64_t p, int chain, uint32_t site) {
  if constexpr (PR_LB_STRESS) {
    // the tag and the word region (a fused pass's iterations each have their own) seed the pauses
    const uint32_t tag = c.tag ^ static_cast<uint32_t>(reinterpret_cast<uintptr_t>(c.lb) >> 8);
    uint32_t h = tag * 0x9E3779B1u ^ static_cast<uint32_t>(p) * 0x85EBCA77u ^ static_cast<uint32_t>(chain) * 0xC2B2AE3Du ^
                 site * 0x27D4EB2Fu;
    h ^= h >> 15;
    h *= 0x2C1B3C6Du;
    h ^= h >> 12;
    const int n = (h & 3) == 0 ? static_cast<int>((h >> 8) & 31) : 0;   // a quarter of the tiles, up to ~100 us
    for (int i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(127);
  } else {
    (void)c; (void)p; (void)chain; (void)site;
  }
}

// The state entering position p in scan order, for the V channels of one lane: the inclusive word of
// position p-1 (the state at the end of its chunk), or, once p-1 has published only its aggregate (the
// chunk's affine map), that map applied to the inclusive word of p-2 -- whichever appears first.  Both are
// the same bits: p-1 publishes its inclusive word as its aggregate applied to its own carry, which by the
// same rule is p-2's inclusive word.  So every carry is the sequential chain apply(aggregate, state), and no
// result depends on timing (a walk that composed several aggregates first would round differently).  The
// walk never goes deeper than one aggregate; forward progress holds because p-1 and p-2 have smaller
// tickets (running or done), and position 0 publishes its inclusive word without waiting.  All V channels
// of the lane wait together: their words were written together by one lane of the predecessor.
template <int S, int V, int TW, int NSLOT>
DEV void lookback_near(const Common& c, const Tile& tl, float (&carry)[V][S]) {
  constexpr int NA = S * S + S;
  const int64_t p1 = tl.p - 1, p2 = tl.p - 2;
  const int q0 = tl.qlane * V;
  bool have_agg = false;   // p-1's aggregate is out (then agg holds it)
  Aff<S> agg[V];
  uint32_t depth = 0;      // 1 once the carry came from an aggregate (counted in stress builds)
  while (true) {
    // a scalar state requests every word a round may use before looking at any (one memory round trip);
    // larger states request p-1's inclusive word, then its aggregate, then p-2's inclusive word, each only
    // while still needed (fewer words live at once: the 2x2 and 4x4 kernels are short of registers)
    uint64_t w1[V][S], wa[V][NA], w2[V][S];
    const bool want_a = !have_agg && p2 >= 0, want_2 = p2 >= 0 && (S == 1 || have_agg);
#pragma unroll
    for (int v = 0; v < V; ++v) {
#pragma unroll
      for (int k = 0; k < S; ++k) w1[v][k] = ld_word(word_at<S, TW, NSLOT>(c, p1, tl.chain, k, q0 + v));
      if (S == 1 && want_a) {
#pragma unroll
        for (int k = 0; k < NA; ++k) wa[v][k] = ld_word(word_at<S, TW, NSLOT>(c, p1, tl.chain, S + k, q0 + v));
      }
      if (S == 1 && want_2) {
#pragma unroll
        for (int k = 0; k < S; ++k) w2[v][k] = ld_word(word_at<S, TW, NSLOT>(c, p2, tl.chain, k, q0 + v));
      }
    }
    bool ok1 = true;
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int k = 0; k < S; ++k) ok1 = ok1 && word_ok(w1[v][k], c.tag);
    if (ok1) {
#pragma unroll
      for (int v = 0; v < V; ++v)
#pragma unroll
        for (int k = 0; k < S; ++k) carry[v][k] = word_val(w1[v][k]);
      break;
    }
    if (want_a) {
      if constexpr (S > 1) {
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
          for (int k = 0; k < NA; ++k) wa[v][k] = ld_word(word_at<S, TW, NSLOT>(c, p1, tl.chain, S + k, q0 + v));
      }
      bool oka = true;
#pragma unroll
      for (int v = 0; v < V; ++v)
#pragma unroll
        for (int k = 0; k < NA; ++k) oka = oka && word_ok(wa[v][k], c.tag);
      if (oka) {
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
          for (int k = 0; k < NA; ++k) aff_set(agg[v], k, word_val(wa[v][k]));
        have_agg = true;
      }
    }
    if (have_agg && (S > 1 || want_2)) {
      if constexpr (S > 1) {
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
          for (int k = 0; k < S; ++k) w2[v][k] = ld_word(word_at<S, TW, NSLOT>(c, p2, tl.chain, k, q0 + v));
      }
      bool ok2 = true;
#pragma unroll
      for (int v = 0; v < V; ++v)
#pragma unroll
        for (int k = 0; k < S; ++k) ok2 = ok2 && word_ok(w2[v][k], c.tag);
      if (ok2) {
#pragma unroll
        for (int v = 0; v < V; ++v) {
          float x[S];
#pragma unroll
          for (int k = 0; k < S; ++k) x[k] = word_val(w2[v][k]);
          apply(agg[v], x);
#pragma unroll
          for (int k = 0; k < S; ++k) carry[v][k] = x[k];
        }
        depth = 1;
        break;
      }
    }
    __builtin_amdgcn_s_sleep(1);
  }
#if PR_LB_STRESS
  atomicMax(&g_lb_max_depth, depth);
#else
  (void)depth;
#endif
}

// The same carry by a walk: each round reads one position's inclusive and aggregate words together,
// starting at p-1; past a position whose aggregate alone is out it moves one back, until it meets an
// inclusive word.  That state is then advanced through the passed aggregates one at a time in scan order
// (re-read: a word never changes once tagged), which is again the chain each tile publishes, bit for
// bit, however deep the walk went.  Nothing is held from one round to the next.
template <int S, int V, int TW, int NSLOT>
DEV void lookback_walk(const Common& c, const Tile& tl, float (&carry)[V][S]) {
  constexpr int NA = S * S + S;
  const int q0 = tl.qlane * V;
  int64_t m = tl.p - 1;   // the position this round looks at
  while (true) {
    uint64_t wi[V][S], wa[V][NA];
#pragma unroll
    for (int v = 0; v < V; ++v) {
#pragma unroll
      for (int k = 0; k < S; ++k) wi[v][k] = ld_word(word_at<S, TW, NSLOT>(c, m, tl.chain, k, q0 + v));
#pragma unroll
      for (int k = 0; k < NA; ++k) wa[v][k] = ld_word(word_at<S, TW, NSLOT>(c, m, tl.chain, S + k, q0 + v));
    }
    bool inc_ok = true, agg_ok = true;
#pragma unroll
    for (int v = 0; v < V; ++v) {
#pragma unroll
      for (int k = 0; k < S; ++k) inc_ok = inc_ok && word_ok(wi[v][k], c.tag);
#pragma unroll
      for (int k = 0; k < NA; ++k) agg_ok = agg_ok && word_ok(wa[v][k], c.tag);
    }
    if (inc_ok) {
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float x[S];
#pragma unroll
        for (int k = 0; k < S; ++k) x[k] = word_val(wi[v][k]);
        // the aggregates of positions m+1 .. p-1, passed on the way, re-read and applied in scan order
        for (int64_t pos = m + 1; pos < tl.p; ++pos) {
          Aff<S> e;
#pragma unroll
          for (int k = 0; k < NA; ++k)
            aff_set(e, k, word_val(ld_word(word_at<S, TW, NSLOT>(c, pos, tl.chain, S + k, q0 + v))));
          apply(e, x);
        }
#pragma unroll
        for (int k = 0; k < S; ++k) carry[v][k] = x[k];
      }
#if PR_LB_STRESS
      atomicMax(&g_lb_max_depth, static_cast<uint32_t>(tl.p - 1 - m));
#endif
      return;
    }
    if (agg_ok) --m;   // pass m (position 0 publishes its inclusive word at once: m stays >= 0)
    else __builtin_amdgcn_s_sleep(1);
  }
}

// the carry of a tile: the walk for the kernels it leaves with fewer registers (the sLSTM Newton
// iteration: 253 VGPRs, two waves per SIMD, against 264 and one wave with lookback_near), else the wait
// at most one aggregate deep
template <int S, int V, int TW, int NSLOT, bool WALK>
DEV void lookback(const Common& c, const Tile& tl, float (&carry)[V][S]) {
  if constexpr (WALK) lookback_walk<S, V, TW, NSLOT>(c, tl, carry);
  else lookback_near<S, V, TW, NSLOT>(c, tl, carry);
}

// max(x, x of another lane) over a DPP lane pattern; rows outside ROWS read 0 (keep x)
template <int CTRL, int ROWS>
DEV uint32_t umax_dpp(uint32_t x) {
  const uint32_t y = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, ROWS, 0xf, false));
  return x > y ? x : y;
}
// nanmax over the wave of values that are >= 0 or a NaN with the sign bit clear (a max of |r|): their
// bit patterns order as unsigned integers the way nanmax orders the values (a NaN above +Inf above
// every finite value), so the wave reduces the bits with integer max.  Lane pairs, quads, half rows
// and rows of 16 by DPP permutes, then row 0's maximum into row 1, row 2's into row 3 and rows 0-1's
// into rows 2-3: lane 63 ends with the wave's maximum, which every lane returns.
DEV float wave_nanmax(float m) {
  uint32_t x = __float_as_uint(m);
  x = umax_dpp<0xb1, 0xf>(x);    // quad_perm [1,0,3,2]
  x = umax_dpp<0x4e, 0xf>(x);    // quad_perm [2,3,0,1]
  x = umax_dpp<0x141, 0xf>(x);   // row_half_mirror
  x = umax_dpp<0x140, 0xf>(x);   // row_mirror
  x = umax_dpp<0x142, 0xa>(x);   // row_bcast:15
  x = umax_dpp<0x143, 0xc>(x);   // row_bcast:31
  return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 63)));
}

// ------------------------------------------------------------------------------------------------
// the generic tile kernel
// ------------------------------------------------------------------------------------------------
template <int S>
DEV Aff<S> shfl_aff(const Aff<S>& m, int src) {
  Aff<S> r;
#pragma unroll
  for (int k = 0; k < S * S; ++k) r.A[k] = __shfl(m.A[k], src, WAVE);
#pragma unroll
  for (int k = 0; k < S; ++k) r.b[k] = __shfl(m.b[k], src, WAVE);
  return r;
}

// the tile of a ticket: its position in scan order, channel group, steps and addressing (the NW
// waves of TS time slices of a workgroup, L steps and V channels per lane)
template <int NW, int TS, int L, int V, bool REV>
DEV void tile_setup(const Common& c, uint32_t ticket, Tile& tl) {
  constexpr int LPR = WAVE / TS, TW = LPR * V;
  tl.lane = threadIdx.x % WAVE;
  tl.wave = threadIdx.x / WAVE;
  tl.slice = tl.lane / LPR;
  tl.qlane = tl.lane % LPR;
  tl.p = ticket / static_cast<uint32_t>(c.n_chains);
  tl.chain = static_cast<int>(ticket % static_cast<uint32_t>(c.n_chains));
  tl.chunk = REV ? c.n_chunks - 1 - tl.p : tl.p;
  tl.t_lo = tl.chunk * static_cast<int64_t>(NW * TS * L) + (tl.wave * TS + tl.slice) * L;
  tl.ch0 = static_cast<int64_t>(tl.chain) * TW + tl.qlane * V;
  tl.active = tl.ch0 < c.C;
  {
    // row b and channel d0 of ch0: the tile's first channel is uniform, so its division is scalar;
    // a lane is less than TW channels further, which wraps into the next row at most once when
    // D >= TW (otherwise a small 32-bit division)
    const int64_t tc0 = static_cast<int64_t>(tl.chain) * TW;
    const int64_t b0 = tc0 / c.D;
    int64_t d = tc0 - b0 * c.D + tl.qlane * V, b = b0;
    if (c.D >= TW) {
      if (d >= c.D) { d -= c.D; ++b; }
    } else {
      const uint32_t q = static_cast<uint32_t>(d) / static_cast<uint32_t>(c.D);
      b += q;
      d -= static_cast<int64_t>(q) * c.D;
    }
    tl.b = tl.active ? b : 0;
    tl.d0 = tl.active ? d : 0;
    // uniform base of the wave (its first slice, the tile's first channel) and the lane's offset;
    // lanes past the last channel read the tile's first channel, like the 64-bit path
    const int wave_u = __builtin_amdgcn_readfirstlane(tl.wave);
    const int64_t t_w = tl.chunk * static_cast<int64_t>(NW * TS * L) + static_cast<int64_t>(wave_u) * TS * L;
    const int64_t d_w = tc0 - b0 * c.D;
    tl.wbase = (b0 * c.T + t_w) * c.D + d_w;
    const int64_t lo = tl.active ? (tl.b - b0) * c.T * c.D + static_cast<int64_t>(tl.slice) * L * c.D + (tl.d0 - d_w)
                                 : static_cast<int64_t>(tl.slice) * L * c.D;
    tl.loff = static_cast<uint32_t>(lo);
  }
  tl.first_seg = tl.wave == 0 && tl.slice == 0;
  tl.last_seg = tl.wave == NW - 1 && tl.slice == TS - 1;
  {
    const int64_t left = c.T - tl.t_lo;
    tl.nvalid = static_cast<int>(left < 0 ? 0 : (left > L ? L : left));
  }
}

// the scan's LDS: each wave's aggregate of its TS*L steps, the state entering each wave's steps (in
// scan order), each wave's max residual
template <class Op>
struct TileShm {
  static constexpr int S = Op::S, NW = Op::NW, TW = (WAVE / Op::TS) * Op::V, NA = S * S + S;
  float (&agg)[NA][NW][TW];
  float (&carry)[S][NW][TW];
  float (&red)[NW];
};
// declares the scan's LDS arrays (and the ticket) in a kernel and the view sh of them
#define PR_TILE_SHM(Op)                                                                           \
  __shared__ uint32_t sh_ticket;                                                                  \
  __shared__ float sh_agg_[TileShm<Op>::NA][TileShm<Op>::NW][TileShm<Op>::TW];                    \
  __shared__ float sh_carry_[TileShm<Op>::S][TileShm<Op>::NW][TileShm<Op>::TW];                   \
  __shared__ float sh_red_[TileShm<Op>::NW];                                                      \
  TileShm<Op> sh{sh_agg_, sh_carry_, sh_red_}

// One scan over the tile's elements ln: each lane's aggregate, the wave's slices, the waves through
// LDS, the look-back across tiles (words of c), and the state entering each lane's steps.  With
// Op::RESID the tile's max of the lanes' rmax goes to res_slot.  Every thread of the workgroup calls
// it (two barriers inside).
template <class Op>
DEV void tile_scan(const typename Op::Args& a, const Common& c, uint32_t* res_slot, const Tile& tl,
                   typename Op::Lane& ln, float rmax, const TileShm<Op>& sh, float (&enter)[Op::V][Op::S]) {
  constexpr int S = Op::S, V = Op::V, L = Op::L, NW = Op::NW, TS = Op::TS, NA = S * S + S;
  constexpr int LPR = WAVE / TS, TW = LPR * V;
  constexpr int NSLOT = Op::NSLOT;
  constexpr bool REV = Op::REVERSE;
  auto& sh_agg = sh.agg;
  auto& sh_carry = sh.carry;
  auto& sh_red = sh.red;
  // per-lane aggregate over its L steps, in scan order; then across the wave's TS slices
  const int q0 = tl.qlane * V;
  const int sp = REV ? TS - 1 - tl.slice : tl.slice;   // the slice's position in scan order
  Aff<S> excl[V];                                      // slices of this wave before mine, composed
#pragma unroll
  for (int v = 0; v < V; ++v) {
    Aff<S> g;
    if constexpr (Op::LANE_AGG) {
      g = ln.agg[v];   // composed by the Op while it produced the elements
    } else {
      g = ln.e[v][REV ? L - 1 : 0];   // the first element itself: no composition with the identity
#pragma unroll
      for (int s = 1; s < L; ++s) g = Op::compose_elem(ln.e[v][REV ? L - 1 - s : s], g);
    }
    excl[v] = aff_id<S>();
    if constexpr (TS > 1) {
      // inclusive scan over slices (Hillis-Steele on lanes LPR apart), then shift by one slice; with two
      // slices the first level's operand already is the earlier slice's inclusive value
      Aff<S> inc = g, prev;
#pragma unroll
      for (int d = 1; d < TS; d <<= 1) {
        const int src = tl.lane + (REV ? d : -d) * LPR;
        const Aff<S> o = shfl_aff(inc, (src + WAVE) % WAVE);
        if (sp >= d) inc = compose(inc, o);
        if (TS == 2) prev = o;
      }
      if constexpr (TS > 2) {
        const int src = tl.lane + (REV ? 1 : -1) * LPR;
        prev = shfl_aff(inc, (src + WAVE) % WAVE);
      }
      if (sp > 0) excl[v] = prev;
      g = inc;
    }
    if (sp == TS - 1) {
#pragma unroll
      for (int k = 0; k < NA; ++k) sh_agg[k][tl.wave][q0 + v] = aff_get(g, k);
    }
  }
  if constexpr (Op::RESID) {
    rmax = wave_nanmax(rmax);
    if (tl.lane == 0) sh_red[tl.wave] = rmax;
  }
  __syncthreads();
  if constexpr (Op::RESID) {
    if (threadIdx.x == 0) {
      uint32_t m = 0u;   // the waves' maxima, >= 0 or NaN: as bits (see wave_nanmax)
#pragma unroll
      for (int w = 0; w < NW; ++w) m = max(m, __float_as_uint(sh_red[w]));
      atomicMax(res_slot, m);
    }
  }

  if (tl.wave == 0 && tl.slice == 0) {
    // one lane per channel group: the tile's aggregate, the look-back, then every wave's entering
    // state (so that each wave reads one value instead of re-composing the waves before it)
    float carry[V][S];
    Aff<S> tagg[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      tagg[v] = aff_id<S>();
#pragma unroll
      for (int s = 0; s < NW; ++s) {
        const int w = REV ? NW - 1 - s : s;
        Aff<S> e;
#pragma unroll
        for (int k = 0; k < NA; ++k) aff_set(e, k, sh_agg[k][w][q0 + v]);
        tagg[v] = compose(e, tagg[v]);
      }
    }
    if (tl.p == 0) {
      Op::init_state(a, tl, carry);
    } else {
      if (tl.active) {
        stress_pause(c, tl.p, tl.chain, 0);
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
          for (int k = 0; k < NA; ++k)
            st_word(word_at<S, TW, NSLOT>(c, tl.p, tl.chain, S + k, q0 + v), c.tag, aff_get(tagg[v], k));
        stress_pause(c, tl.p, tl.chain, 1);
        lookback<S, V, TW, NSLOT, Op::LB_WALK>(c, tl, carry);
      } else {
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
          for (int k = 0; k < S; ++k) carry[v][k] = 0.0f;
      }
    }
    if (tl.active && tl.p + 1 < c.n_chunks) {
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float x[S];
#pragma unroll
        for (int k = 0; k < S; ++k) x[k] = carry[v][k];
        apply(tagg[v], x);
#pragma unroll
        for (int k = 0; k < S; ++k) st_word(word_at<S, TW, NSLOT>(c, tl.p, tl.chain, k, q0 + v), c.tag, x[k]);
      }
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      float x[S];
#pragma unroll
      for (int k = 0; k < S; ++k) x[k] = carry[v][k];
#pragma unroll
      for (int s = 0; s < NW; ++s) {
        const int w = REV ? NW - 1 - s : s;
#pragma unroll
        for (int k = 0; k < S; ++k) sh_carry[k][w][q0 + v] = x[k];
        if (s + 1 < NW) {
          Aff<S> e;
#pragma unroll
          for (int k = 0; k < NA; ++k) aff_set(e, k, sh_agg[k][w][q0 + v]);
          apply(e, x);
        }
      }
    }
  }
  __syncthreads();

  // state entering this lane's steps: the wave's entering state advanced through earlier slices
#pragma unroll
  for (int v = 0; v < V; ++v) {
    float xv[S];
#pragma unroll
    for (int k = 0; k < S; ++k) xv[k] = sh_carry[k][tl.wave][q0 + v];
    if constexpr (TS > 1) apply(excl[v], xv);
#pragma unroll
    for (int k = 0; k < S; ++k) enter[v][k] = xv[k];
  }
}

// The residual part of tile_scan alone, for a launch whose elements all have A = 0 (a Picard sweep: every
// state is its own element's b, so no scan and no look-back are needed): the tile's max of the lanes' rmax
// goes to res_slot.  Every thread of the workgroup calls it (one barrier inside).
template <class Op>
DEV void tile_resid(uint32_t* res_slot, const Tile& tl, float rmax, const TileShm<Op>& sh) {
  constexpr int NW = Op::NW;
  auto& sh_red = sh.red;
  rmax = wave_nanmax(rmax);
  if (tl.lane == 0) sh_red[tl.wave] = rmax;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) m = max(m, __float_as_uint(sh_red[w]));
    atomicMax(res_slot, m);
  }
}

template <class Op>
DEV uint32_t* op_res_slot(const typename Op::Args& a) {
  if constexpr (Op::RESID) return a.res_slot;
  else return nullptr;
}

// One tile per workgroup; LOOP: each workgroup takes tickets until none is left, so the grid need only hold
// what can be resident (for launches that usually find the solve stopped and exit at once: a grid of one
// workgroup per tile costs ~15 us to dispatch even then).  Tickets still go out in scan order, and a tile
// waits only on smaller tickets, held by running workgroups or done, so neither form can deadlock.
template <class Op, bool LOOP = false>
__global__ __launch_bounds__(Op::NW * WAVE) __attribute__((amdgpu_waves_per_eu(Op::MINW)))
void k_tile(const typename Op::Args a) {
  constexpr int S = Op::S, V = Op::V, L = Op::L, NW = Op::NW, TS = Op::TS;
  static_assert(TS == 1 || TS == 2 || TS == 4, "time slices per wave");
  PR_TILE_SHM(Op);

  if (Op::skip(a)) return;  // uniform: decided from values written by earlier launches
  const Common& c = a.c;
  while (true) {
    if (threadIdx.x == 0)
      sh_ticket = __hip_atomic_fetch_add(c.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if constexpr (LOOP) {
      if (sh_ticket >= static_cast<uint32_t>(c.n_chains) * static_cast<uint32_t>(c.n_chunks)) return;
    }
    Tile tl;
    tile_setup<NW, TS, L, V, Op::REVERSE>(c, sh_ticket, tl);

    typename Op::Lane ln;
    const float rmax = Op::produce(a, tl, ln);
    float x[V][S];
    if (Op::pointwise(a)) {   // uniform
      // each element is (0, f): the state entering a lane only ever meets a zero A, and apply gives f for
      // any finite state, exactly as the scan would
      tile_resid<Op>(op_res_slot<Op>(a), tl, rmax, sh);
#pragma unroll
      for (int v = 0; v < V; ++v)
#pragma unroll
        for (int k = 0; k < S; ++k) x[v][k] = 0.0f;
    } else {
      tile_scan<Op>(a, c, op_res_slot<Op>(a), tl, ln, rmax, sh, x);
    }
    Op::finish(a, tl, ln, x);
    if constexpr (!LOOP) return;
    __syncthreads();   // the tile's shared memory and ticket are free again
  }
}

// ------------------------------------------------------------------------------------------------
// cells: value, Jacobian, and (for the VJP) the partials needed by the gate gradients
// ------------------------------------------------------------------------------------------------
template <int CELL> struct CellInfo;
template <> struct CellInfo<CELL_LINEAR> { static constexpr int S = 1, G = 2; };
template <> struct CellInfo<CELL_GRU> { static constexpr int S = 1, G = 3; };
template <> struct CellInfo<CELL_LSTM> { static constexpr int S = 2, G = 4; };
template <> struct CellInfo<CELL_SLSTM> { static constexpr int S = 4, G = 4; };

// Per-lane channel parameters for V channels: the recurrent weights w and biases b, and the same
// two scaled by the exponent factor of their gate (-log2(e) for a sigmoid gate, 2 log2(e) for a tanh
// gate), so that a gate's exp2 argument is fma(sw, h, fma(scale, U, sb)) = scale * (U + w h + b).
template <int G, int V>
struct Params {
  float w[G][V], bias[G][V], sw[G][V], sb[G][V];
};
template <int CELL> DEV float gate_scale(int g);
template <> DEV float gate_scale<CELL_GRU>(int g) { return g == 2 ? 2.0f * kLog2e : -kLog2e; }     // z, r, c
template <> DEV float gate_scale<CELL_LSTM>(int g) { return g == 3 ? 2.0f * kLog2e : -kLog2e; }    // i, f, o, g
template <> DEV float gate_scale<CELL_SLSTM>(int) { return 1.0f; }   // used unscaled (log domain)
template <> DEV float gate_scale<CELL_LINEAR>(int) { return 0.0f; }

template <int CELL, int G, int V>
DEV void load_params(const float* w, const float* bias, int64_t D, int64_t d0, Params<G, V>& pm) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
    ldv_param<V>(w, g * D + d0, pm.w[g]);
    ldv_param<V>(bias, g * D + d0, pm.bias[g]);
    const float sc = gate_scale<CELL>(g);
#pragma unroll
    for (int v = 0; v < V; ++v) {
      pm.sw[g][v] = sc * pm.w[g][v];
      pm.sb[g][v] = sc * pm.bias[g][v];
    }
  }
}

// the part of gate g's exponent argument that does not depend on the state, scale * (U + b): the cells
// add sw * h (GRU candidate: sw * r h) to it
template <int CELL, int G, int V>
DEV float gate_in(const Params<G, V>& pm, int g, int v, float u) {
  return fmaf(gate_scale<CELL>(g), u, pm.sb[g][v]);
}

// sigmoid and tanh of a pre-scaled exponent argument x (see Params)
DEV float sig_x(float x) { return hw_rcp(1.0f + hw_exp2(x)); }
DEV float tanh_x(float x) { return fmaf(-2.0f, hw_rcp(1.0f + hw_exp2(x)), 1.0f); }

// GRU: z = sig(U_z + a_z h + b_z), r = sig(U_r + a_r h + b_r), c = tanh(U_c + a_c r h + b_c),
//      h' = (1 - z) h + z c,  J = (1 - z) + (c - h) z (1 - z) a_z + z (1 - c^2) a_c (r + h r (1 - r) a_r)
//      gate partials: d h'/d u_z = (c - h) z (1 - z), d h'/d u_c = z (1 - c^2),
//                     d h'/d u_r = d h'/d u_c a_c h r (1 - r)
struct GruOut {
  float f, J, pz, pc, r;
};
// the cell from its gates' state-independent arguments a = gate_in(U)
template <int G, int V>
DEV GruOut gru_eval_in(const Params<G, V>& pm, int v, float az, float ar, float ac, float h) {
  GruOut o;
  const float z = sig_x(fmaf(pm.sw[0][v], h, az));
  const float r = sig_x(fmaf(pm.sw[1][v], h, ar));
  const float rh = r * h;
  const float c = tanh_x(fmaf(pm.sw[2][v], rh, ac));
  const float cmh = c - h;
  o.f = fmaf(z, cmh, h);
  const float zz = fmaf(-z, z, z);                    // z (1 - z)
  const float hrr = fmaf(-r, rh, rh);                 // h r (1 - r)
  o.pc = z * fmaf(-c, c, 1.0f);                       // z (1 - c^2)
  o.pz = cmh * zz;
  o.r = r;
  o.J = fmaf(o.pc * pm.w[2][v], fmaf(hrr, pm.w[1][v], r), fmaf(o.pz, pm.w[0][v], 1.0f - z));
  return o;
}
template <int G, int V>
DEV GruOut gru_eval(const Params<G, V>& pm, int v, float uz, float ur, float uc, float h) {
  return gru_eval_in(pm, v, gate_in<CELL_GRU>(pm, 0, v, uz), gate_in<CELL_GRU>(pm, 1, v, ur),
                     gate_in<CELL_GRU>(pm, 2, v, uc), h);
}

// LSTM: i, f, o = sig(U + w h + b), g = tanh(U_g + w_g h + b_g), c' = f c + i g, h' = o tanh(c')
struct LstmPart {
  float c2, h2;           // new state
  float J00, J01, J10, J11;
  float dc_i, dc_f, dc_g; // d c' / d u_{i,f,g}
  float dh_o, kh;         // d h' / d u_o, d h' / d c'
};
template <int G, int V>
DEV LstmPart lstm_eval_in(const Params<G, V>& pm, int v, float ai, float af, float ao, float ag, float c, float h) {
  LstmPart p;
  const float ig = sig_x(fmaf(pm.sw[0][v], h, ai));
  const float fg = sig_x(fmaf(pm.sw[1][v], h, af));
  const float og = sig_x(fmaf(pm.sw[2][v], h, ao));
  const float gg = tanh_x(fmaf(pm.sw[3][v], h, ag));
  p.c2 = fmaf(fg, c, ig * gg);
  const float tc = tanh_x(2.0f * kLog2e * p.c2);
  p.h2 = og * tc;
  p.dc_i = gg * fmaf(-ig, ig, ig);
  p.dc_f = c * fmaf(-fg, fg, fg);
  p.dc_g = ig * fmaf(-gg, gg, 1.0f);
  p.kh = og * fmaf(-tc, tc, 1.0f);
  p.dh_o = tc * fmaf(-og, og, og);
  const float dc_dh = fmaf(p.dc_i, pm.w[0][v], fmaf(p.dc_f, pm.w[1][v], p.dc_g * pm.w[3][v]));
  p.J00 = fg;
  p.J01 = dc_dh;
  p.J10 = p.kh * fg;
  p.J11 = fmaf(p.dh_o, pm.w[2][v], p.kh * dc_dh);
  return p;
}
template <int G, int V>
DEV LstmPart lstm_eval(const Params<G, V>& pm, int v, float ui, float uf, float uo, float ug, float c, float h) {
  return lstm_eval_in(pm, v, gate_in<CELL_LSTM>(pm, 0, v, ui), gate_in<CELL_LSTM>(pm, 1, v, uf),
                      gate_in<CELL_LSTM>(pm, 2, v, uo), gate_in<CELL_LSTM>(pm, 3, v, ug), c, h);
}

// sLSTM, diagonal recurrence, state (c, n, m, h), gates z, i, f, o (the published sLSTM with
// exponential input gate, sigmoid forget gate and log-domain stabiliser m):
//   u_g = U_g + w_g h + b_g, z = tanh(u_z), o = sig(u_o), lf = log sig(u_f),
//   m' = max(lf + m, u_i), i' = exp(u_i - m'), f' = exp(lf + m - m'),
//   c' = f' c + i' z, n' = f' n + i', h' = o c' / n'.
// At a tie of the max the forget branch is taken (its derivative is the branch's).
// J is row-major over (c, n, m, h); d[i][g] = d s'_i / d u_g (gate order z, i, f, o).
struct SlstmPart {
  float s2[4];
  float J[16];
  float d[16];
};
template <int G, int V>
DEV SlstmPart slstm_eval(const Params<G, V>& pm, int v, float Uz, float Ui, float Uf, float Uo, float c, float n,
                         float m, float h) {
  SlstmPart p;
  const float uz = fmaf(pm.w[0][v], h, Uz + pm.bias[0][v]);
  const float ui = fmaf(pm.w[1][v], h, Ui + pm.bias[1][v]);
  const float uf = fmaf(pm.w[2][v], h, Uf + pm.bias[2][v]);
  const float uo = fmaf(pm.w[3][v], h, Uo + pm.bias[3][v]);
  const float z = tanh_x(2.0f * kLog2e * uz);
  const float o = sig_x(-kLog2e * uo);
  // log sig(u_f) = min(u_f, 0) - log(1 + e^{-|u_f|}); d/du_f = sig(-u_f)
  const float e = hw_exp2(-kLog2e * fabsf(uf));
  const float lf = fminf(uf, 0.0f) - kLn2 * __builtin_amdgcn_logf(1.0f + e);
  const float dlf = uf >= 0.0f ? e * hw_rcp(1.0f + e) : hw_rcp(1.0f + e);
  const float lfm = lf + m;
  const bool fb = lfm >= ui;
  const float m2 = fb ? lfm : ui;
  const float ip = hw_exp2(kLog2e * (ui - m2)), fp = hw_exp2(kLog2e * (lfm - m2));
  const float c2 = fmaf(fp, c, ip * z), n2 = fmaf(fp, n, ip);
  const float rn = hw_rcp(n2);
  const float hn = c2 * rn;                 // c' / n'
  p.s2[0] = c2; p.s2[1] = n2; p.s2[2] = m2; p.s2[3] = o * hn;
  // i', f', m' as functions of (u_i, u_f, m) on the active branch
  const float dm_ui = fb ? 0.0f : 1.0f, dm_uf = fb ? dlf : 0.0f, dm_m = fb ? 1.0f : 0.0f;
  const float dip_ui = ip * (1.0f - dm_ui), dip_uf = -ip * dm_uf, dip_m = -ip * dm_m;
  const float dfp_ui = -fp * dm_ui, dfp_uf = fp * (dlf - dm_uf), dfp_m = fp * (1.0f - dm_m);
  const float dc[4] = {ip * fmaf(-z, z, 1.0f), fmaf(c, dfp_ui, z * dip_ui), fmaf(c, dfp_uf, z * dip_uf), 0.0f};
  const float dn[4] = {0.0f, fmaf(n, dfp_ui, dip_ui), fmaf(n, dfp_uf, dip_uf), 0.0f};
  const float dm[4] = {0.0f, dm_ui, dm_uf, 0.0f};
  const float orn = o * rn;
  float dh[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) dh[g] = orn * fmaf(-hn, dn[g], dc[g]);   // o (dc n' - c' dn) / n'^2
  dh[3] += hn * fmaf(-o, o, o);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    p.d[0 * 4 + g] = dc[g]; p.d[1 * 4 + g] = dn[g]; p.d[2 * 4 + g] = dm[g]; p.d[3 * 4 + g] = dh[g];
  }
  const float dc_m = fmaf(c, dfp_m, z * dip_m), dn_m = fmaf(n, dfp_m, dip_m);
  float sc = 0.0f, sn = 0.0f, sm = 0.0f, sh = 0.0f;   // h enters every gate through w_g h
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    sc = fmaf(dc[g], pm.w[g][v], sc);
    sn = fmaf(dn[g], pm.w[g][v], sn);
    sm = fmaf(dm[g], pm.w[g][v], sm);
    sh = fmaf(dh[g], pm.w[g][v], sh);
  }
  p.J[0] = fp;   p.J[1] = 0.0f; p.J[2] = dc_m;  p.J[3] = sc;
  p.J[4] = 0.0f; p.J[5] = fp;   p.J[6] = dn_m;  p.J[7] = sn;
  p.J[8] = 0.0f; p.J[9] = 0.0f; p.J[10] = dm_m; p.J[11] = sm;
  p.J[12] = orn * fp;                       // d h' / d c
  p.J[13] = -orn * hn * fp;                 // d h' / d n
  p.J[14] = orn * fmaf(-hn, dn_m, dc_m);    // d h' / d m
  p.J[15] = sh;
  return p;
}

// running max of |r| by the NaN-propagating maximum (gfx950's v_maximum3_f32 takes two steps' |r| per
// instruction); the result is NaN iff some r was NaN or infinite
struct ResidMax {
  float m = 0.0f;
  DEV void add(float r) { m = __builtin_elementwise_maximum(m, fabsf(r)); }
  DEV float get() const { return m <= 3.40282347e+38f ? m : __builtin_nanf(""); }
};

template <int S, int V>
DEV void load_s0(const float* s0, int64_t B, int64_t D, const Tile& tl, float (&x)[V][S]) {
#pragma unroll
  for (int k = 0; k < S; ++k) {
    float t[V];
    if (s0 && tl.active) {
      ldv<V, DT_F32>(s0, (k * B + tl.b) * D + tl.d0, t);
    } else {
#pragma unroll
      for (int v = 0; v < V; ++v) t[v] = 0.0f;
    }
#pragma unroll
    for (int v = 0; v < V; ++v) x[v][k] = t[v];
  }
}

// ------------------------------------------------------------------------------------------------
// Op 1: linear recurrence (pararnn_linear_scan)
// ------------------------------------------------------------------------------------------------
template <int S_, int DT, bool REV, int V_, int L_, int NW_, int MINW_, int TS_, bool SEG = false>
struct LinearOp {
  static constexpr int S = S_, V = V_, L = L_, NW = NW_, MINW = MINW_, TS = TS_;
  static constexpr bool REVERSE = REV, RESID = false, LB_WALK = false, LANE_AGG = false;
  static constexpr int NSLOT = S + S * S + S;
  struct Args {
    Common c;
    const void* a;
    const void* b;
    const float* s0;
    float* out;
    int64_t B;
    uint32_t* res_slot;  // unused
  };
  struct Lane {
    Aff<S> e[V][L];
  };
  static DEV bool skip(const Args&) { return false; }
  static DEV bool pointwise(const Args&) { return false; }
  static constexpr uint32_t EMASK = kFullMask<S>;
  static DEV Aff<S> compose_elem(const Aff<S>& e, const Aff<S>& g) { return compose_masked<S, EMASK>(e, g); }
  static DEV void init_state(const Args& a, const Tile& tl, float (&x)[V][S]) {
    load_s0<S, V>(a.s0, a.B, a.c.D, tl, x);
  }
  // Lanes past the last channel load channel 0 (valid addresses) and are never published or
  // stored; steps past T use clamped addresses and become identity elements (MASKED path only).
  static DEV float produce(const Args& a, const Tile& tl, Lane& ln) {
    if (tl.nvalid == L) produce_t<false>(a, tl, ln);
    else produce_t<true>(a, tl, ln);
    return 0.0f;
  }
  template <bool MASKED>
  static DEV void produce_t(const Args& a, const Tile& tl, Lane& ln) {
    const int64_t D = a.c.D, T = a.c.T, N = a.c.N, row = tl.b * T;
    float av[S * S][L][V], bv[S][L][V];
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int64_t t = MASKED ? clamp_t(tl.t_lo + i, T) : tl.t_lo + i;
      const int64_t idx = (row + t) * D + tl.d0;
#pragma unroll
      for (int k = 0; k < S * S; ++k) ldv<V, DT>(a.a, k * N + idx, av[k][i]);
#pragma unroll
      for (int k = 0; k < S; ++k) ldv<V, DT>(a.b, k * N + idx, bv[k][i]);
    }
    // packed sequences: no state crosses into a sequence's first step (forward) or out of its
    // first step into the previous sequence's last (reverse), so that step's A is zero
    uint32_t sb = 0;
    if constexpr (SEG) sb = seg_bits(a.c.seg, tl.t_lo + (REV ? 1 : 0), T);
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const bool ok = !MASKED || i < tl.nvalid;
      const bool rs = SEG && ((sb >> i) & 1u);
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const Aff<S> one = aff_id<S>();
#pragma unroll
        for (int k = 0; k < S * S; ++k) ln.e[v][i].A[k] = ok ? (rs ? 0.0f : av[k][i][v]) : one.A[k];
#pragma unroll
        for (int k = 0; k < S; ++k) ln.e[v][i].b[k] = ok ? bv[k][i][v] : 0.0f;
      }
    }
  }
  static DEV void finish(const Args& a, const Tile& tl, Lane& ln, float (&x)[V][S]) {
    if (!tl.active) return;
    const int64_t base = (tl.b * a.c.T + tl.t_lo) * a.c.D + tl.d0;
#pragma unroll
    for (int s = 0; s < L; ++s) {
      const int i = REV ? L - 1 - s : s;
      if (i >= tl.nvalid) continue;
#pragma unroll
      for (int v = 0; v < V; ++v) apply_masked<S, EMASK>(ln.e[v][i], x[v]);
#pragma unroll
      for (int k = 0; k < S; ++k) {
        float o[V];
#pragma unroll
        for (int v = 0; v < V; ++v) o[v] = x[v][k];
        stv<V>(a.out + k * a.c.N + base + i * a.c.D, o);
      }
    }
  }
};

// ------------------------------------------------------------------------------------------------
// Op 2: one fused Newton iteration (pararnn_newton_solve)
//   element of step t:  A_t = J_t,  b_t = f_t - J_t h^k_{t-1}   (f_t, J_t at (h^k_{t-1}, x_t))
//   so that the scan gives h^{k+1}_t = h^k_t + delta_t with delta_t = J_t delta_{t-1} - r_t,
//   r_t = h^k_t - f_t (the same iterate, written without forming delta).  The max |r_t| is
//   reduced for the tolerance test.  LINEAR: the element is (a_t, b_t) itself.
// ------------------------------------------------------------------------------------------------
template <int CELL, int DT, int V_, int L_, int NW_, int MINW_, int TS_, bool SEG = false>
struct NewtonOp {
  static constexpr int S = CellInfo<CELL>::S, G = CellInfo<CELL>::G;
  static constexpr int V = V_, L = L_, NW = NW_, MINW = MINW_, TS = TS_;
  static constexpr bool REVERSE = false, RESID = true, LANE_AGG = false;
  static constexpr bool LB_WALK = CELL == CELL_SLSTM;   // see lookback
  static constexpr bool FUSABLE = CELL == CELL_GRU || CELL == CELL_LSTM;   // k_fused is built for these
  static constexpr int HALO = S + S * S + S;          // slot of the halo words
  static constexpr int NSLOT = HALO + S;
  struct Args {
    Common c;
    const void* pre[4];
    const float* w;
    const float* bias;
    const float* s0;
    const float* h_in;        // H^k [S][B][T][D], or NULL for H^k = 0 (or the warm start)
    float* h_out;             // H^{k+1}; may equal h_in
    int32_t warm;             // h_in == NULL: H^0_t = f(0, x_t) computed here instead of 0
    int32_t picard;           // this launch is a Picard sweep: H^{k+1}_t = f(H^k_{t-1}, x_t) (A = 0)
    uint32_t* res_slot;       // max |r| of this iteration (float bits, atomicMax)
    const uint32_t* res_hist; // max |r| of earlier iterations
    int32_t k;
    float tol;
    int64_t B;
  };
  struct Lane {
    Aff<S> e[V][L];
  };
  static DEV bool pointwise(const Args& a) { return a.picard != 0; }   // a Picard sweep: elements (0, f)
  static DEV bool skip(const Args& a) {
    if (!(a.tol > 0.0f)) return false;
    for (int j = 0; j < a.k; ++j) {
      const float r = __uint_as_float(a.res_hist[j]);
      if (!(r >= a.tol) || r == INFINITY) return true;  // converged, or NaN / Inf: stop
    }
    return false;
  }
  static constexpr uint32_t EMASK = CELL == CELL_SLSTM ? kSlstmJMask : kFullMask<S>;   // elements are J_t
  static DEV Aff<S> compose_elem(const Aff<S>& e, const Aff<S>& g) { return compose_masked<S, EMASK>(e, g); }
  static DEV void init_state(const Args& a, const Tile& tl, float (&x)[V][S]) {
    load_s0<S, V>(a.s0, a.B, a.c.D, tl, x);
  }
  static DEV float produce(const Args& a, const Tile& tl, Lane& ln) {
    if (a.picard) return tl.nvalid == L ? produce_t<false, true>(a, tl, ln) : produce_t<true, true>(a, tl, ln);
    return tl.nvalid == L ? produce_t<false, false>(a, tl, ln) : produce_t<true, false>(a, tl, ln);
  }
  // f(0, u) for channel slot v (pararnn-torch README, "Method": the GRU / LSTM warm start)
  static DEV void warm_state(const Params<G, V>& pm, int v, const float (&u)[G][V], float (&o)[S]) {
    if constexpr (CELL == CELL_LINEAR) {
      o[0] = u[1][v];
    } else if constexpr (CELL == CELL_GRU) {
      o[0] = gru_eval(pm, v, u[0][v], u[1][v], u[2][v], 0.0f).f;
    } else if constexpr (CELL == CELL_LSTM) {
      const LstmPart q = lstm_eval(pm, v, u[0][v], u[1][v], u[2][v], u[3][v], 0.0f, 0.0f);
      o[0] = q.c2;
      o[1] = q.h2;
    } else {
      const SlstmPart q = slstm_eval(pm, v, u[0][v], u[1][v], u[2][v], u[3][v], 0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
      for (int k = 0; k < S; ++k) o[k] = q.s2[k];
    }
  }
  // one lane's inputs of an iteration: the current iterate at steps t_lo-1 .. t_lo+L-1 (h[.][0] is the
  // step before the lane's first), the gate inputs of its L steps, its channels' parameters and the
  // packed-sequence start bits of its steps
  struct Regs {
    float h[S][L + 1][V];
    float u[G][L][V];
    Params<G, V> pm;
    uint32_t sb;
  };
  // a lane's gate inputs as 32-bit words (the fused pass parks them in LDS between iterations).  The first
  // NPRE gates are kept as their state-independent arguments gate_in (fp32, the same single fma the cell
  // does at every iteration, done once), as far as LDS leaves room for two workgroups per CU: all gates of
  // fp32 inputs and of the LSTM, the first gate of the bf16 GRU.  The others as read: two bf16 values a
  // word -- exact, since they were read as bf16 -- or one fp32 value.
  static constexpr int NPRE = CELL == CELL_GRU ? (DT == DT_BF16 ? 1 : G) : (CELL == CELL_LSTM ? G : 0);
  static constexpr int NRAW = G - NPRE;
  static constexpr int PWORDS = NPRE * L * V;
  static constexpr int UWORDS = PWORDS + (DT == DT_BF16 ? (NRAW * L * V + 1) / 2 : NRAW * L * V);
  static DEV void pack_u(const Regs& rg, uint32_t (&w)[UWORDS]) {
#pragma unroll
    for (int g = 0; g < NPRE; ++g)
#pragma unroll
      for (int i = 0; i < L; ++i)
#pragma unroll
        for (int v = 0; v < V; ++v)
          w[(g * L + i) * V + v] = __float_as_uint(gate_in<CELL>(rg.pm, g, v, rg.u[g][i][v]));
    const float* u = &rg.u[NPRE][0][0];
    constexpr int NR = NRAW * L * V;
    if constexpr (DT == DT_BF16) {
#pragma unroll
      for (int q = 0; q < UWORDS - PWORDS; ++q) {
        const uint32_t lo = __float_as_uint(u[2 * q]) >> 16;
        const uint32_t hi = 2 * q + 1 < NR ? __float_as_uint(u[2 * q + 1]) & 0xffff0000u : 0u;
        w[PWORDS + q] = hi | lo;
      }
    } else {
#pragma unroll
      for (int q = 0; q < NR; ++q) w[PWORDS + q] = __float_as_uint(u[q]);
    }
  }
  // gate input (g >= NPRE, step i, channel slot v) from the words of pack_u, word q at w[q]
  template <class Words>
  static DEV float unpack_u(const Words& w, int g, int i, int v) {
    const int f = ((g - NPRE) * L + i) * V + v;
    if constexpr (DT == DT_BF16) {
      const uint32_t x = w[PWORDS + (f >> 1)];
      return __uint_as_float((f & 1) ? (x & 0xffff0000u) : (x << 16));
    } else {
      return __uint_as_float(w[PWORDS + f]);
    }
  }
  // gate_in of gate g at step i, channel slot v from the words of pack_u
  template <class Words>
  static DEV float unpack_in(const Words& w, const Params<G, V>& pm, int g, int i, int v) {
    if (g < NPRE) return __uint_as_float(w[(g * L + i) * V + v]);
    return gate_in<CELL>(pm, g, v, unpack_u(w, g, i, v));
  }
  template <bool MASKED, bool PIC>
  static DEV float produce_t(const Args& a, const Tile& tl, Lane& ln) {
    Regs rg;
    load<MASKED>(a, tl, rg);
    return elements<MASKED, PIC>(tl, rg, ln, RegU{rg});
  }
  // gate input (g, step i, channel slot v) from the lane's registers, and its gate_in
  struct RegU {
    const Regs& rg;
    DEV float operator()(int g, int i, int v) const { return rg.u[g][i][v]; }
    DEV float in(const Params<G, V>& pm, int g, int i, int v) const { return gate_in<CELL>(pm, g, v, rg.u[g][i][v]); }
  };
  template <bool MASKED>
  static DEV void load(const Args& a, const Tile& tl, Regs& rg) {
    const int64_t D = a.c.D, T = a.c.T, N = a.c.N, row = tl.b * T;
    const Common& c = a.c;
    constexpr int TW = (WAVE / TS) * V;
    const int q0 = tl.qlane * V;
    const bool have_h = a.h_in != nullptr;
    // loads first, all of them
    float (&h)[S][L + 1][V] = rg.h;
    float (&u)[G][L][V] = rg.u;
    const bool fast = !MASKED && c.off32 && (S == 1 || PR_FAST_S2);   // uniform
    if (have_h && fast) {
      // one descriptor per state plane at the wave's step before its first; step i is i+1 rows on
      // (the base may lie before the plane when the wave starts at t = 0: that halo is not loaded)
      const uint32_t vo = tl.loff * 4u, row_b = static_cast<uint32_t>(D) * 4u;
#pragma unroll
      for (int k = 0; k < S; ++k) {
        const Rsrc r = rsrc_at(a.h_in + (k * N + tl.wbase - D));
#pragma unroll
        for (int i = 0; i < L; ++i) ldv_buf<V, DT_F32>(r, vo, (i + 1) * row_b, h[k][i + 1]);
        if (!tl.first_seg) ldv_buf<V, DT_F32>(r, vo, 0u, h[k][0]);
      }
    } else if (have_h) {
#pragma unroll
      for (int i = 0; i < L; ++i) {
        const int64_t t = MASKED ? clamp_t(tl.t_lo + i, T) : tl.t_lo + i;
#pragma unroll
        for (int k = 0; k < S; ++k) ldv<V, DT_F32>(a.h_in, k * N + (row + t) * D + tl.d0, h[k][i + 1]);
      }
      if (!tl.first_seg) {
        // h^k_{t_lo-1} lies in this tile's chunk (written only after the tile's look-back)
        const int64_t idx = (row + clamp_t(tl.t_lo - 1, T)) * D + tl.d0;
#pragma unroll
        for (int k = 0; k < S; ++k) ldv<V, DT_F32>(a.h_in, k * N + idx, h[k][0]);
      }
    } else {
#pragma unroll
      for (int i = 0; i <= L; ++i)
#pragma unroll
        for (int k = 0; k < S; ++k)
#pragma unroll
          for (int v = 0; v < V; ++v) h[k][i][v] = 0.0f;
    }
    if (fast) {
      constexpr uint32_t ESZ = DT == DT_F32 ? 4u : 2u;
      const uint32_t vo = tl.loff * ESZ, row_b = static_cast<uint32_t>(D) * ESZ;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const Rsrc r = rsrc_at(static_cast<const char*>(a.pre[g]) + tl.wbase * ESZ);
#pragma unroll
        for (int i = 0; i < L; ++i) ldv_buf<V, DT>(r, vo, i * row_b, u[g][i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < L; ++i) {
        const int64_t t = MASKED ? clamp_t(tl.t_lo + i, T) : tl.t_lo + i;
#pragma unroll
        for (int g = 0; g < G; ++g) ldv<V, DT>(a.pre[g], (row + t) * D + tl.d0, u[g][i]);
      }
    }
    Params<G, V>& pm = rg.pm;
    if constexpr (CELL != CELL_LINEAR) load_params<CELL, G, V>(a.w, a.bias, D, tl.d0, pm);
    if (!have_h && a.warm) {
      // warm first iterate: every step's state is the cell applied to a zero previous state, so
      // h^0_{t_lo-1} needs only that step's gate inputs (no halo exchange in this iteration)
      float up[G][V];
      const int64_t tp = clamp_t(tl.t_lo - 1, T);
#pragma unroll
      for (int g = 0; g < G; ++g) ldv<V, DT>(a.pre[g], (row + tp) * D + tl.d0, up[g]);
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float o[S];
        warm_state(pm, v, up, o);
#pragma unroll
        for (int k = 0; k < S; ++k) h[k][0][v] = o[k];
#pragma unroll
        for (int i = 0; i < L; ++i) {
          float ui[G][V];
#pragma unroll
          for (int g = 0; g < G; ++g) ui[g][v] = u[g][i][v];
          warm_state(pm, v, ui, o);
#pragma unroll
          for (int k = 0; k < S; ++k) h[k][i + 1][v] = o[k];
        }
      }
    }
    if (tl.t_lo == 0) {
      float x[V][S];
      load_s0<S, V>(a.s0, a.B, D, tl, x);
#pragma unroll
      for (int k = 0; k < S; ++k)
#pragma unroll
        for (int v = 0; v < V; ++v) h[k][0][v] = x[v][k];
    }
    if (have_h && tl.active) {
      // publish this tile's last state (the h^k the next tile's first step needs), then take the
      // previous tile's: the trajectory is updated in place, so it cannot be re-read from memory
      if (tl.last_seg && tl.nvalid == L && tl.p + 1 < c.n_chunks) {
        stress_pause(c, tl.p, tl.chain, 2);
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
          for (int k = 0; k < S; ++k)
            st_word(word_at<S, TW, NSLOT>(c, tl.p, tl.chain, HALO + k, q0 + v), c.tag, h[k][L][v]);
      }
      if (tl.first_seg && tl.t_lo != 0) {
        // every halo word of the lane in flight at once (one memory round trip, not one per word);
        // the predecessor publishes them right after its loads, so a retry is rare
        uint64_t wv[V][S];
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
          for (int k = 0; k < S; ++k) wv[v][k] = ld_word(word_at<S, TW, NSLOT>(c, tl.p - 1, tl.chain, HALO + k, q0 + v));
        bool ok = false;
        while (!ok) {
          ok = true;
#pragma unroll
          for (int v = 0; v < V; ++v)
#pragma unroll
            for (int k = 0; k < S; ++k) ok = ok && word_ok(wv[v][k], c.tag);
          if (!ok) {
            __builtin_amdgcn_s_sleep(1);
#pragma unroll
            for (int v = 0; v < V; ++v)
#pragma unroll
              for (int k = 0; k < S; ++k)
                if (!word_ok(wv[v][k], c.tag)) wv[v][k] = ld_word(word_at<S, TW, NSLOT>(c, tl.p - 1, tl.chain, HALO + k, q0 + v));
          }
        }
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
          for (int k = 0; k < S; ++k) h[k][0][v] = word_val(wv[v][k]);
      }
    }
    // packed sequences: a step that begins a sequence starts from the zero state, so its previous
    // state is 0 and its Jacobian (the element's A) is zero
    rg.sb = 0;
    if constexpr (SEG) rg.sb = seg_bits(c.seg, tl.t_lo, T);
  }
  // the scan elements of the lane's steps at the iterate in rg, and the max residual over its valid steps;
  // the gate inputs come from uin(g, i, v), fetched step by step
  template <bool MASKED, bool PIC, class UIn>
  static DEV float elements(const Tile& tl, const Regs& rg, Lane& ln, const UIn& uin) {
    const float (&h)[S][L + 1][V] = rg.h;
    const Params<G, V>& pm = rg.pm;
    ResidMax rm;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const bool ok = !MASKED || i < tl.nvalid;
      const bool rs = SEG && ((rg.sb >> i) & 1u);
      // the GRU and LSTM take each gate's gate_in, the linear cell and the sLSTM the inputs themselves
      float ui[G][V];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int v = 0; v < V; ++v) {
          if constexpr (CELL == CELL_GRU || CELL == CELL_LSTM) ui[g][v] = uin.in(pm, g, i, v);
          else ui[g][v] = uin(g, i, v);
        }
#pragma unroll
      for (int v = 0; v < V; ++v) {
        Aff<S> e;
        // a Picard sweep keeps f and drops the Jacobian: the element is (0, f)
        if constexpr (CELL == CELL_LINEAR) {
          const float hp = rs ? 0.0f : h[0][i][v];
          const float f = fmaf(ui[0][v], hp, ui[1][v]);
          if (ok) rm.add(h[0][i + 1][v] - f);
          e.A[0] = (rs || PIC) ? 0.0f : ui[0][v];
          e.b[0] = PIC ? f : ui[1][v];
        } else if constexpr (CELL == CELL_GRU) {
          const float hp = rs ? 0.0f : h[0][i][v];
          const GruOut q = gru_eval_in(pm, v, ui[0][v], ui[1][v], ui[2][v], hp);
          if (ok) rm.add(h[0][i + 1][v] - q.f);
          e.A[0] = (rs || PIC) ? 0.0f : q.J;
          e.b[0] = PIC ? q.f : fmaf(-q.J, hp, q.f);
        } else if constexpr (CELL == CELL_LSTM) {
          const float cp = rs ? 0.0f : h[0][i][v], hp = rs ? 0.0f : h[1][i][v];
          const LstmPart q = lstm_eval_in(pm, v, ui[0][v], ui[1][v], ui[2][v], ui[3][v], cp, hp);
          if (ok) {
            rm.add(h[0][i + 1][v] - q.c2);
            rm.add(h[1][i + 1][v] - q.h2);
          }
          e.A[0] = (rs || PIC) ? 0.0f : q.J00;
          e.A[1] = (rs || PIC) ? 0.0f : q.J01;
          e.A[2] = (rs || PIC) ? 0.0f : q.J10;
          e.A[3] = (rs || PIC) ? 0.0f : q.J11;
          e.b[0] = PIC ? q.c2 : q.c2 - fmaf(q.J00, cp, q.J01 * hp);
          e.b[1] = PIC ? q.h2 : q.h2 - fmaf(q.J10, cp, q.J11 * hp);
        } else {
          float sp[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) sp[k] = rs ? 0.0f : h[k][i][v];
          const SlstmPart q = slstm_eval(pm, v, ui[0][v], ui[1][v], ui[2][v], ui[3][v], sp[0], sp[1],
                                         sp[2], sp[3]);
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (ok) rm.add(h[k][i + 1][v] - q.s2[k]);
#pragma unroll
          for (int k = 0; k < 16; ++k) e.A[k] = (rs || PIC) ? 0.0f : q.J[k];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float acc = q.s2[r];
            if (!PIC) {
#pragma unroll
              for (int k = 0; k < 4; ++k) acc = fmaf(-q.J[r * 4 + k], sp[k], acc);
            }
            e.b[r] = acc;
          }
        }
        if (MASKED) {
          const Aff<S> one = aff_id<S>();
#pragma unroll
          for (int k = 0; k < S * S; ++k) ln.e[v][i].A[k] = ok ? e.A[k] : one.A[k];
#pragma unroll
          for (int k = 0; k < S; ++k) ln.e[v][i].b[k] = ok ? e.b[k] : 0.0f;
        } else {
          ln.e[v][i] = e;
        }
      }
    }
    return tl.active ? rm.get() : 0.0f;
  }
  // the update of finish kept in registers instead of stored: rg.h[.][i+1] becomes H^{k+1} at the
  // lane's step i (the same multiply-adds in the same order).  Steps past T take the last state: the
  // next iteration masks them, and writing every register ends the old values' lives here.
  template <bool MASKED>
  static DEV void advance(const Tile& tl, const Lane& ln, float (&x)[V][S], Regs& rg) {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      if (!MASKED || i < tl.nvalid) {   // an unmasked launch has every step of every lane
#pragma unroll
        for (int v = 0; v < V; ++v) apply_masked<S, EMASK>(ln.e[v][i], x[v]);
      }
#pragma unroll
      for (int k = 0; k < S; ++k)
#pragma unroll
        for (int v = 0; v < V; ++v) rg.h[k][i + 1][v] = x[v][k];
    }
  }
  // the re-run of a speculative fused pass of m iterations from iteration a.k (tolerance mode): the
  // iterations the solve really runs from there, j + 1 for the first j < m - 1 whose residual met the
  // stop rule of skip, or 0 when none did (then the pass's result stands)
  static DEV int redo_count(const Args& a, int m) {
    for (int j = 0; j + 1 < m; ++j) {
      const float r = __uint_as_float(a.res_hist[a.k + j]);
      if (!(r >= a.tol) || r == INFINITY) return j + 1;
    }
    return 0;
  }
  static DEV void finish(const Args& a, const Tile& tl, Lane& ln, float (&x)[V][S]) {
    if (!tl.active) return;
    const int64_t base = (tl.b * a.c.T + tl.t_lo) * a.c.D + tl.d0;
    const bool fast = a.c.off32 && tl.nvalid == L;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      if (i >= tl.nvalid) continue;
#pragma unroll
      for (int v = 0; v < V; ++v) apply_masked<S, EMASK>(ln.e[v][i], x[v]);
#pragma unroll
      for (int k = 0; k < S; ++k) {
        float o[V];
#pragma unroll
        for (int v = 0; v < V; ++v) o[v] = x[v][k];
        if (fast) stv_u<V>(a.h_out, k * a.c.N + tl.wbase + i * a.c.D, tl.loff, o);
        else stv<V>(a.h_out + k * a.c.N + base + i * a.c.D, o);
      }
    }
  }
};

// ------------------------------------------------------------------------------------------------
// Op 3: VJP by one reverse scan (pararnn_scan_vjp)
//   element of step t:  A_t = J_{t+1}^T (0 at t = T-1),  b_t = e_h g_t   ->  lambda_t
//   then dU_{gate,t} = lambda_t . d f/d u_gate at (s_{t-1}, x_t), and per-tile parameter partials.
// ------------------------------------------------------------------------------------------------
template <int CELL> struct VjpStash;
template <> struct VjpStash<CELL_LINEAR> { float hp; };
template <> struct VjpStash<CELL_GRU> { float pz, pc, hp, r; };
template <> struct VjpStash<CELL_LSTM> { float dci, dcf, dcg, dho, kh, hp; };

struct VjpArgs {
  Common c;
  const void* pre[4];
  const float* w;
  const float* bias;
  const float* s0;
  const float* s;       // trajectory [S][B][T][D]
  const float* g;       // [B][T][D]
  float* d_pre;         // [G][B][T][D]
  float* lambda_out;    // [S][B][T][D] or NULL
  float* d_s0;          // [S][B][D] or NULL
  float* partial;       // [n_chunks][NPAR][C]
  int64_t B;
  uint32_t* res_slot;   // unused
};

// the diagonal cells with a state of one or two (the sLSTM: SlstmVjpOp below)
template <int CELL, int DT, int V_, int L_, int NW_, int MINW_, int TS_, bool SEG = false>
struct VjpOp {
  static_assert(CELL != CELL_SLSTM, "the sLSTM VJP is SlstmVjpOp");
  static constexpr int S = CellInfo<CELL>::S, G = CellInfo<CELL>::G;
  static constexpr int V = V_, L = L_, NW = NW_, MINW = MINW_, TS = TS_;
  static constexpr bool REVERSE = true, RESID = false, LB_WALK = false, LANE_AGG = false;
  static constexpr int NSLOT = S + S * S + S;
  static constexpr int NPAR = CELL == CELL_LINEAR ? 0 : 2 * G;  // dw[G], dbias[G] partial sums
  using Args = VjpArgs;
  struct Lane {
    Aff<S> e[V][L];
    VjpStash<CELL> st[V][L];
    float J0[V][S * S];   // Jacobian at step 0 (only used by the lane that owns t = 0)
    float ac[V];          // GRU: a_c, for d h'/d u_r
  };
  static DEV bool skip(const Args&) { return false; }
  static DEV bool pointwise(const Args&) { return false; }
  static constexpr uint32_t EMASK = kFullMask<S>;   // elements are J_{t+1}^T
  static DEV Aff<S> compose_elem(const Aff<S>& e, const Aff<S>& g) { return compose_masked<S, EMASK>(e, g); }
  static DEV void init_state(const Args&, const Tile&, float (&x)[V][S]) {
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int k = 0; k < S; ++k) x[v][k] = 0.0f;   // nothing flows in from beyond the last step
  }
  static DEV float produce(const Args& a, const Tile& tl, Lane& ln) {
    // the unmasked path needs every step and the next lane's first step inside [0, T)
    if (tl.t_lo + L < a.c.T) produce_t<false>(a, tl, ln);
    else produce_t<true>(a, tl, ln);
    return 0.0f;
  }
  template <bool MASKED>
  static DEV void produce_t(const Args& a, const Tile& tl, Lane& ln) {
    const int64_t D = a.c.D, T = a.c.T, N = a.c.N, row = tl.b * T;
    // loads first: evaluation e (0..L) is the cell step at t = t_lo + e, which needs U_t and
    // s_{t-1}; e = L belongs to the next lane's first step and only contributes its Jacobian
    float u[G][L + 1][V], sp[S][L + 1][V], gv[L][V];
    if (!MASKED && a.c.off32) {   // uniform
      // as NewtonOp::load: one buffer descriptor per plane at the wave's base element, the lane's 32-bit
      // offset, and the step's row offset as a uniform operand (no vector address arithmetic per load).
      // s_{t-1} comes from a descriptor one row before the base; its first row only where t_lo > 0 (the
      // lane at t = 0 takes s0 below, and its row would lie before the plane).  (The linear scan's loads
      // ran no faster this way.)
      constexpr uint32_t ESZ = DT == DT_F32 ? 4u : 2u;
      const uint32_t row_u = static_cast<uint32_t>(D) * ESZ, row_f = static_cast<uint32_t>(D) * 4u;
      const uint32_t vu = tl.loff * ESZ, vf = tl.loff * 4u;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const Rsrc r = rsrc_at(static_cast<const char*>(a.pre[g]) + tl.wbase * ESZ);
#pragma unroll
        for (int e = 0; e <= L; ++e) ldv_buf<V, DT>(r, vu, e * row_u, u[g][e]);
      }
#pragma unroll
      for (int k = 0; k < S; ++k) {
        const Rsrc r = rsrc_at(a.s + (k * N + tl.wbase - D));
#pragma unroll
        for (int e = 1; e <= L; ++e) ldv_buf<V, DT_F32>(r, vf, e * row_f, sp[k][e]);
        if (tl.t_lo > 0) {
          ldv_buf<V, DT_F32>(r, vf, 0u, sp[k][0]);
        } else {
#pragma unroll
          for (int v = 0; v < V; ++v) sp[k][0][v] = 0.0f;
        }
      }
      const Rsrc rg = rsrc_at(a.g + tl.wbase);
#pragma unroll
      for (int e = 0; e < L; ++e) ldv_buf<V, DT_F32>(rg, vf, e * row_f, gv[e]);
    } else {
#pragma unroll
      for (int e = 0; e <= L; ++e) {
        const int64_t idx = (row + (MASKED ? clamp_t(tl.t_lo + e, T) : tl.t_lo + e)) * D + tl.d0;
        const int64_t idp = (row + clamp_t(tl.t_lo + e - 1, T)) * D + tl.d0;
#pragma unroll
        for (int g = 0; g < G; ++g) ldv<V, DT>(a.pre[g], idx, u[g][e]);
#pragma unroll
        for (int k = 0; k < S; ++k) ldv<V, DT_F32>(a.s, k * N + idp, sp[k][e]);
        if (e < L) ldv<V, DT_F32>(a.g, idx, gv[e]);
      }
    }
    if (tl.t_lo == 0) {
      float x[V][S];
      load_s0<S, V>(a.s0, a.B, D, tl, x);
#pragma unroll
      for (int k = 0; k < S; ++k)
#pragma unroll
        for (int v = 0; v < V; ++v) sp[k][0][v] = x[v][k];
    }
    Params<G, V> pm;
    if constexpr (CELL != CELL_LINEAR) load_params<CELL, G, V>(a.w, a.bias, D, tl.d0, pm);
    if constexpr (CELL == CELL_GRU) {
#pragma unroll
      for (int v = 0; v < V; ++v) ln.ac[v] = pm.w[2][v];
    }
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int k = 0; k < S * S; ++k) ln.J0[v][k] = 0.0f;
    // packed sequences: evaluation e at a sequence's first step starts from the zero state, and its
    // Jacobian is zero (no adjoint flows back into the previous sequence)
    uint32_t sb = 0;
    if constexpr (SEG) sb = seg_bits(a.c.seg, tl.t_lo, T);
    if constexpr (SEG) {
#pragma unroll
      for (int e = 0; e <= L; ++e)
#pragma unroll
        for (int k = 0; k < S; ++k)
#pragma unroll
          for (int v = 0; v < V; ++v) sp[k][e][v] = ((sb >> e) & 1u) ? 0.0f : sp[k][e][v];
    }
    // evaluations e = L .. 0; the element of step e takes the (transposed) Jacobian of e + 1
    float Jn[V][S * S];
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int k = 0; k < S * S; ++k) Jn[v][k] = 0.0f;
#pragma unroll
    for (int e = L; e >= 0; --e) {
      const bool ok = !MASKED || e < tl.nvalid || (e == L && tl.t_lo + L < T);
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float J[S * S];
        VjpStash<CELL> st{};
        if constexpr (CELL == CELL_LINEAR) {
          J[0] = u[0][e][v];
          st.hp = sp[0][e][v];
        } else if constexpr (CELL == CELL_GRU) {
          const GruOut q = gru_eval(pm, v, u[0][e][v], u[1][e][v], u[2][e][v], sp[0][e][v]);
          J[0] = q.J;
          st.pz = q.pz;
          st.pc = q.pc;
          st.hp = sp[0][e][v];
          st.r = q.r;
        } else if constexpr (CELL == CELL_LSTM) {
          const LstmPart q = lstm_eval(pm, v, u[0][e][v], u[1][e][v], u[2][e][v], u[3][e][v], sp[0][e][v],
                                       sp[1][e][v]);
          J[0] = q.J00; J[1] = q.J01; J[2] = q.J10; J[3] = q.J11;
          st.dci = q.dc_i; st.dcf = q.dc_f; st.dcg = q.dc_g; st.dho = q.dh_o; st.kh = q.kh;
          st.hp = sp[1][e][v];
        }
        if (e < L) {
          const bool okl = !MASKED || e < tl.nvalid;
          Aff<S>& el = ln.e[v][e];
          // A = J_{t+1}^T (zero past the last step), b = e_h g_t; identity for masked steps
#pragma unroll
          for (int i = 0; i < S; ++i)
#pragma unroll
            for (int j = 0; j < S; ++j) el.A[i * S + j] = okl ? Jn[v][j * S + i] : (i == j ? 1.0f : 0.0f);
#pragma unroll
          for (int k = 0; k < S; ++k) el.b[k] = 0.0f;
          el.b[S - 1] = okl ? gv[e][v] : 0.0f;
          ln.st[v][e] = st;
          if (e == 0 && tl.t_lo == 0) {
#pragma unroll
            for (int k = 0; k < S * S; ++k) ln.J0[v][k] = J[k];
          }
        }
        const bool live = ok && !(SEG && ((sb >> e) & 1u));
#pragma unroll
        for (int k = 0; k < S * S; ++k) Jn[v][k] = live ? J[k] : 0.0f;
      }
    }
  }
  static DEV void finish(const Args& a, const Tile& tl, Lane& ln, float (&x)[V][S]) {
    constexpr int TW = (WAVE / TS) * V, NSEG = NW * TS;
    constexpr int NP = NPAR > 0 ? NPAR : 1;
    __shared__ float sh_par[NP][NSEG][TW];
    const int64_t D = a.c.D, T = a.c.T, N = a.c.N;
    float par[V][NP];
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int j = 0; j < NP; ++j) par[v][j] = 0.0f;
    if (tl.active) {
      const int64_t base = (tl.b * T + tl.t_lo) * D + tl.d0;
#pragma unroll
      for (int s = 0; s < L; ++s) {
        const int i = L - 1 - s;
        const int64_t t = tl.t_lo + i;
        if (t >= T) continue;
        float du[G][V], lam[S][V];
#pragma unroll
        for (int v = 0; v < V; ++v) {
          apply_masked<S, EMASK>(ln.e[v][i], x[v]);
          const VjpStash<CELL>& st = ln.st[v][i];
#pragma unroll
          for (int k = 0; k < S; ++k) lam[k][v] = x[v][k];
          if constexpr (CELL == CELL_LINEAR) {
            du[0][v] = x[v][0] * st.hp;
            du[1][v] = x[v][0];
          } else if constexpr (CELL == CELL_GRU) {
            const float l = x[v][0];
            const float ac = ln.ac[v];
            du[0][v] = l * st.pz;
            du[2][v] = l * st.pc;
            du[1][v] = du[2][v] * ac * st.hp * st.r * (1.0f - st.r);
            par[v][0] = fmaf(du[0][v], st.hp, par[v][0]);
            par[v][1] = fmaf(du[1][v], st.hp, par[v][1]);
            par[v][2] = fmaf(du[2][v], st.r * st.hp, par[v][2]);
#pragma unroll
            for (int g = 0; g < 3; ++g) par[v][3 + g] += du[g][v];
          } else if constexpr (CELL == CELL_LSTM) {
            const float lc = x[v][0], lh = x[v][1];
            const float m = fmaf(st.kh, lh, lc);   // lambda_c + kh lambda_h
            du[0][v] = m * st.dci;
            du[1][v] = m * st.dcf;
            du[2][v] = lh * st.dho;
            du[3][v] = m * st.dcg;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              par[v][g] = fmaf(du[g][v], st.hp, par[v][g]);
              par[v][4 + g] += du[g][v];
            }
          }
          if (t == 0 && a.d_s0) {
#pragma unroll
            for (int i2 = 0; i2 < S; ++i2) {
              float acc = 0.0f;
#pragma unroll
              for (int j = 0; j < S; ++j) acc = fmaf(ln.J0[v][j * S + i2], x[v][j], acc);
              a.d_s0[(i2 * a.B + tl.b) * D + tl.d0 + v] = acc;
            }
          }
        }
        if (a.c.off32) {   // uniform: the plane's base element plus the lane's 32-bit offset
          const int64_t ub = tl.wbase + i * D;
#pragma unroll
          for (int g = 0; g < G; ++g) stv_u<V>(a.d_pre, g * N + ub, tl.loff, du[g]);
          if (a.lambda_out) {
#pragma unroll
            for (int k = 0; k < S; ++k) stv_u<V>(a.lambda_out, k * N + ub, tl.loff, lam[k]);
          }
        } else {
          const int64_t idx = base + i * D;
#pragma unroll
          for (int g = 0; g < G; ++g) stv<V>(a.d_pre + g * N + idx, du[g]);
          if (a.lambda_out) {
#pragma unroll
            for (int k = 0; k < S; ++k) stv<V>(a.lambda_out + k * N + idx, lam[k]);
          }
        }
      }
    }
    if constexpr (NPAR > 0) {
      const int q0 = tl.qlane * V, seg = tl.wave * TS + tl.slice;
#pragma unroll
      for (int v = 0; v < V; ++v)
#pragma unroll
        for (int j = 0; j < NPAR; ++j) sh_par[j][seg][q0 + v] = par[v][j];
      __syncthreads();
      // fixed-order sum over the waves of the tile
      for (int idx = threadIdx.x; idx < NPAR * TW; idx += NW * WAVE) {
        const int j = idx / TW, q = idx % TW;
        const int64_t ch = static_cast<int64_t>(tl.chain) * TW + q;
        if (ch >= a.c.C) continue;
        float sum = 0.0f;
        for (int w = 0; w < NSEG; ++w) sum += sh_par[j][w][q];
        a.partial[(tl.chunk * NPAR + j) * a.c.C + ch] = sum;
      }
    }
  }
};

// The sLSTM VJP (same elements and epilogue as VjpOp) with the cell evaluated twice instead of kept: a
// step's element (a 4x4 transposed Jacobian and b) and its 16 gate partials are 37 values, and holding
// them from the scan to the re-walk limits a lane to 4 steps at two waves per SIMD.  Here a lane keeps
// only its inputs (4 gate and 4 state values a step, the upstream gradient), composes its elements into
// its aggregate while it produces them, and evaluates the cell again in the re-walk for the partials and
// the Jacobian.  That leaves room for 12 steps a lane, which spreads the scan's per-lane work (the slice
// scan, the waves' aggregates, the look-back) over three times as many steps.
template <int DT, int V_, int L_, int NW_, int MINW_, int TS_, bool SEG = false>
struct SlstmVjpOp {
  static constexpr int S = 4, G = 4;
  static constexpr int V = V_, L = L_, NW = NW_, MINW = MINW_, TS = TS_;
  static constexpr bool REVERSE = true, RESID = false, LB_WALK = false, LANE_AGG = true;
  static constexpr int NSLOT = S + S * S + S;
  static constexpr int NPAR = 2 * G;                 // dw[G], dbias[G] partial sums
  static constexpr uint32_t EMASK = kSlstmJtMask;    // elements are J_{t+1}^T
  using Args = VjpArgs;
  struct Lane {
    Aff<S> agg[V];                               // the lane's elements composed in scan order
    float u[G][L + 1][V], sp[S][L + 1][V];       // U_t and s_{t-1} of steps t_lo .. t_lo + L
    float gv[L][V];                              // the upstream gradient of steps t_lo .. t_lo + L - 1
    uint32_t sb;                                 // packed sequences: sequence-start bits of those steps
  };
  static DEV bool skip(const Args&) { return false; }
  static DEV bool pointwise(const Args&) { return false; }
  static DEV Aff<S> compose_elem(const Aff<S>& e, const Aff<S>& g) { return compose_masked<S, EMASK>(e, g); }
  static DEV void init_state(const Args&, const Tile&, float (&x)[V][S]) {
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int k = 0; k < S; ++k) x[v][k] = 0.0f;   // nothing flows in from beyond the last step
  }

  // the element of step e: A = J_{e+1}^T (Jn: zero past the last step or at a sequence start), b = e_h g_e;
  // the identity where step e is masked
  static DEV Aff<S> element(const float (&Jn)[S * S], float g, bool okl) {
    Aff<S> el;
#pragma unroll
    for (int i = 0; i < S; ++i)
#pragma unroll
      for (int j = 0; j < S; ++j) el.A[i * S + j] = okl ? Jn[j * S + i] : (i == j ? 1.0f : 0.0f);
#pragma unroll
    for (int k = 0; k < S; ++k) el.b[k] = 0.0f;
    el.b[S - 1] = okl ? g : 0.0f;
    return el;
  }
  template <int V2>
  static DEV SlstmPart eval(const Params<G, V2>& pm, const Lane& ln, int v, int e) {
    return slstm_eval(pm, v, ln.u[0][e][v], ln.u[1][e][v], ln.u[2][e][v], ln.u[3][e][v], ln.sp[0][e][v],
                      ln.sp[1][e][v], ln.sp[2][e][v], ln.sp[3][e][v]);
  }
  // whether evaluation e (0..L) takes part: steps inside [0, T), and e = L only where the next lane's
  // first step exists; and whether its Jacobian reaches back (not at a sequence start)
  template <bool MASKED>
  static DEV bool ok_at(const Args& a, const Tile& tl, int e) {
    return !MASKED || e < tl.nvalid || (e == L && tl.t_lo + L < a.c.T);
  }
  static DEV bool live_at(const Lane& ln, int e) { return !(SEG && ((ln.sb >> e) & 1u)); }

  static DEV float produce(const Args& a, const Tile& tl, Lane& ln) {
    if (tl.t_lo + L < a.c.T) produce_t<false>(a, tl, ln);
    else produce_t<true>(a, tl, ln);
    return 0.0f;
  }
  template <bool MASKED>
  static DEV void produce_t(const Args& a, const Tile& tl, Lane& ln) {
    const int64_t D = a.c.D, T = a.c.T, N = a.c.N, row = tl.b * T;
#pragma unroll
    for (int e = 0; e <= L; ++e) {
      const int64_t idx = (row + (MASKED ? clamp_t(tl.t_lo + e, T) : tl.t_lo + e)) * D + tl.d0;
      const int64_t idp = (row + clamp_t(tl.t_lo + e - 1, T)) * D + tl.d0;
#pragma unroll
      for (int g = 0; g < G; ++g) ldv<V, DT>(a.pre[g], idx, ln.u[g][e]);
#pragma unroll
      for (int k = 0; k < S; ++k) ldv<V, DT_F32>(a.s, k * N + idp, ln.sp[k][e]);
      if (e < L) ldv<V, DT_F32>(a.g, idx, ln.gv[e]);
    }
    if (tl.t_lo == 0) {
      float x[V][S];
      load_s0<S, V>(a.s0, a.B, D, tl, x);
#pragma unroll
      for (int k = 0; k < S; ++k)
#pragma unroll
        for (int v = 0; v < V; ++v) ln.sp[k][0][v] = x[v][k];
    }
    ln.sb = 0;
    if constexpr (SEG) {
      ln.sb = seg_bits(a.c.seg, tl.t_lo, T);
#pragma unroll
      for (int e = 0; e <= L; ++e)
#pragma unroll
        for (int k = 0; k < S; ++k)
#pragma unroll
          for (int v = 0; v < V; ++v) ln.sp[k][e][v] = ((ln.sb >> e) & 1u) ? 0.0f : ln.sp[k][e][v];
    }
    Params<G, V> pm;
    load_params<CELL_SLSTM, G, V>(a.w, a.bias, D, tl.d0, pm);
    // evaluations e = L .. 0; the element of step e takes the Jacobian of e + 1, and the lane's aggregate
    // composes them in scan order (step L - 1 first)
#pragma unroll
    for (int v = 0; v < V; ++v) {
      float Jn[S * S];
#pragma unroll
      for (int e = L; e >= 0; --e) {
        const SlstmPart q = eval(pm, ln, v, e);
        if (e < L) {
          const Aff<S> el = element(Jn, ln.gv[e][v], !MASKED || e < tl.nvalid);
          ln.agg[v] = e == L - 1 ? el : compose_elem(el, ln.agg[v]);
        }
        const bool live = ok_at<MASKED>(a, tl, e) && live_at(ln, e);
#pragma unroll
        for (int k = 0; k < S * S; ++k) Jn[k] = live ? q.J[k] : 0.0f;
      }
    }
  }

  static DEV void finish(const Args& a, const Tile& tl, Lane& ln, float (&x)[V][S]) {
    constexpr int TW = (WAVE / TS) * V, NSEG = NW * TS;
    __shared__ float sh_par[NPAR][NSEG][TW];
    float par[V][NPAR];
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int j = 0; j < NPAR; ++j) par[v][j] = 0.0f;
    if (tl.active) {
      if (tl.t_lo + L < a.c.T) walk<false>(a, tl, ln, x, par);
      else walk<true>(a, tl, ln, x, par);
    }
    const int q0 = tl.qlane * V, seg = tl.wave * TS + tl.slice;
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int j = 0; j < NPAR; ++j) sh_par[j][seg][q0 + v] = par[v][j];
    __syncthreads();
    // fixed-order sum over the waves of the tile
    for (int idx = threadIdx.x; idx < NPAR * TW; idx += NW * WAVE) {
      const int j = idx / TW, q = idx % TW;
      const int64_t ch = static_cast<int64_t>(tl.chain) * TW + q;
      if (ch >= a.c.C) continue;
      float sum = 0.0f;
      for (int w = 0; w < NSEG; ++w) sum += sh_par[j][w][q];
      a.partial[(tl.chunk * NPAR + j) * a.c.C + ch] = sum;
    }
  }
  // the re-walk from the state entering the lane (lambda after its last step), steps L-1 .. 0: each step's
  // cell again (its partials, and its Jacobian for the step before), lambda_t, dU_t and the parameter sums
  template <bool MASKED>
  static DEV void walk(const Args& a, const Tile& tl, Lane& ln, float (&x)[V][S], float (&par)[V][NPAR]) {
    const int64_t D = a.c.D, N = a.c.N;
    const int64_t base = (tl.b * a.c.T + tl.t_lo) * D + tl.d0;
    Params<G, V> pm;
    load_params<CELL_SLSTM, G, V>(a.w, a.bias, D, tl.d0, pm);
    float Jn[V][S * S];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const SlstmPart q = eval(pm, ln, v, L);
      const bool live = ok_at<MASKED>(a, tl, L) && live_at(ln, L);
#pragma unroll
      for (int k = 0; k < S * S; ++k) Jn[v][k] = live ? q.J[k] : 0.0f;
    }
#pragma unroll
    for (int s = 0; s < L; ++s) {
      const int i = L - 1 - s;
      if (MASKED && i >= tl.nvalid) {   // past T: an identity element, no output; J_i reaches nothing
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
          for (int k = 0; k < S * S; ++k) Jn[v][k] = 0.0f;
        continue;
      }
      const int64_t t = tl.t_lo + i;
      float du[G][V], lam[S][V];
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const SlstmPart q = eval(pm, ln, v, i);
        apply_masked<S, EMASK>(element(Jn[v], ln.gv[i][v], true), x[v]);
#pragma unroll
        for (int k = 0; k < S; ++k) lam[k][v] = x[v][k];
        const float hp = ln.sp[3][i][v];
        // dU_g = sum_i lambda_i d s'_i / d u_g; every gate's w multiplies h_{t-1}
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float acc = 0.0f;
#pragma unroll
          for (int i2 = 0; i2 < 4; ++i2) acc = fmaf(x[v][i2], q.d[i2 * 4 + g], acc);
          du[g][v] = acc;
          par[v][g] = fmaf(acc, hp, par[v][g]);
          par[v][4 + g] += acc;
        }
        if (t == 0 && a.d_s0) {
#pragma unroll
          for (int i2 = 0; i2 < S; ++i2) {
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < S; ++j) acc = fmaf(q.J[j * S + i2], x[v][j], acc);
            a.d_s0[(i2 * a.B + tl.b) * D + tl.d0 + v] = acc;
          }
        }
        const bool live = live_at(ln, i);
#pragma unroll
        for (int k = 0; k < S * S; ++k) Jn[v][k] = live ? q.J[k] : 0.0f;
      }
      const int64_t idx = base + i * D;
#pragma unroll
      for (int g = 0; g < G; ++g) stv<V>(a.d_pre + g * N + idx, du[g]);
      if (a.lambda_out) {
#pragma unroll
        for (int k = 0; k < S; ++k) stv<V>(a.lambda_out + k * N + idx, lam[k]);
      }
    }
  }
};

// ------------------------------------------------------------------------------------------------
// Fused Newton pass: iterations k .. k+m-1 of a tile in one launch (diagonal GRU and LSTM).  The tile
// loads its gate inputs and the first iterate once and keeps the trajectory in registers from one
// iteration to the next; only the last iteration writes it.  Each iteration is the element, scan and
// update arithmetic of one k_tile<NewtonOp> launch, with look-back words of its own (region j).  The
// state before a lane's first step is the value the lane of the previous segment computed -- by a
// shuffle within the wave, through LDS across waves, by a halo word across tiles -- which is what
// k_tile reads back from memory, so the trajectory equals m launches of k_tile bit for bit.
// Deadlock freedom is k_tile's: tiles take tickets in scan order, and a tile waits only on tiles with
// smaller tickets, each of which is resident or done.
// ------------------------------------------------------------------------------------------------
struct FuseArgs {
  int32_t m;        // iterations of this launch
  int32_t redo;     // nonzero: re-run of a speculative pass (NewtonOp::redo_count decides, uniformly)
  int64_t region;   // look-back words from one iteration's region to the next
};

// A lane's gate inputs in LDS (lane-minor words of NewtonOp::pack_u), read where the element loop uses them.
template <class Op>
struct LdsU {
  const uint32_t (*sh_u)[Op::NW * WAVE];
  struct Col {
    const uint32_t (*sh_u)[Op::NW * WAVE];
    DEV uint32_t operator[](int q) const { return sh_u[q][threadIdx.x]; }
  };
  DEV float operator()(int g, int i, int v) const { return Op::unpack_u(Col{sh_u}, g, i, v); }
  template <class P>
  DEV float in(const P& pm, int g, int i, int v) const { return Op::unpack_in(Col{sh_u}, pm, g, i, v); }
};

// The lane's channel parameters back from LDS at the start of every iteration of a fused pass.  The empty
// asm is a compiler memory barrier (no instruction): no read of the parked gate inputs or parameters is
// merged with the stores before the loop, so no value derived from them is hoisted out of it to occupy
// registers across the scans.
template <class Op>
DEV void fused_inputs(const Tile& tl, const float (*sh_pm)[4][(WAVE / Op::TS) * Op::V], typename Op::Regs& rg) {
  constexpr int G = Op::G, V = Op::V;
  asm volatile("" ::: "memory");
  const int q0 = tl.qlane * V;
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int v = 0; v < V; ++v) {
      rg.pm.w[g][v] = sh_pm[g][0][q0 + v];
      rg.pm.bias[g][v] = sh_pm[g][1][q0 + v];
      rg.pm.sw[g][v] = sh_pm[g][2][q0 + v];
      rg.pm.sb[g][v] = sh_pm[g][3][q0 + v];
    }
}

// Before iteration j >= 1 of a fused pass: the state before the lane's first step at the new iterate
// (chunk 0's first lane keeps s0): the previous slice's last state by a shuffle, the previous wave's
// through LDS, the previous tile's from its halo word in region c.
template <class Op>
DEV void fused_enter(const Common& c, const Tile& tl, const float (*sh_last)[Op::NW][(WAVE / Op::TS) * Op::V],
                     typename Op::Regs& rg) {
  constexpr int S = Op::S, V = Op::V, L = Op::L, TS = Op::TS;
  constexpr int LPR = WAVE / TS, TW = LPR * V, NSLOT = Op::NSLOT;
  const int q0 = tl.qlane * V;
  float prev[S][V];
#pragma unroll
  for (int k = 0; k < S; ++k)
#pragma unroll
    for (int v = 0; v < V; ++v) prev[k][v] = __shfl(rg.h[k][L][v], (tl.lane - LPR + WAVE) % WAVE, WAVE);
  if (tl.slice > 0) {
#pragma unroll
    for (int k = 0; k < S; ++k)
#pragma unroll
      for (int v = 0; v < V; ++v) rg.h[k][0][v] = prev[k][v];
  } else if (tl.wave > 0) {
#pragma unroll
    for (int k = 0; k < S; ++k)
#pragma unroll
      for (int v = 0; v < V; ++v) rg.h[k][0][v] = sh_last[k][tl.wave - 1][q0 + v];
  } else if (tl.t_lo != 0 && tl.active) {
    uint64_t wv[V][S];
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int k = 0; k < S; ++k) wv[v][k] = ld_word(word_at<S, TW, NSLOT>(c, tl.p - 1, tl.chain, Op::HALO + k, q0 + v));
    bool ok = false;
    while (!ok) {
      ok = true;
#pragma unroll
      for (int v = 0; v < V; ++v)
#pragma unroll
        for (int k = 0; k < S; ++k) ok = ok && word_ok(wv[v][k], c.tag);
      if (!ok) {
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
          for (int k = 0; k < S; ++k)
            if (!word_ok(wv[v][k], c.tag))
              wv[v][k] = ld_word(word_at<S, TW, NSLOT>(c, tl.p - 1, tl.chain, Op::HALO + k, q0 + v));
      }
    }
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int k = 0; k < S; ++k) rg.h[k][0][v] = word_val(wv[v][k]);
  }
}

// After iteration j < m-1: this lane's last state for the next iteration, to the next tile's first lane
// (halo word of region j+1, `region` words on from c) and the next wave's first slice (LDS); ends with a
// barrier so that the LDS values are visible.
template <class Op>
DEV void fused_leave(const Common& c, int64_t region, const Tile& tl,
                     float (*sh_last)[Op::NW][(WAVE / Op::TS) * Op::V], const typename Op::Regs& rg) {
  constexpr int S = Op::S, V = Op::V, L = Op::L, TS = Op::TS;
  constexpr int LPR = WAVE / TS, TW = LPR * V, NSLOT = Op::NSLOT;
  const int q0 = tl.qlane * V;
  if (tl.last_seg && tl.active && tl.nvalid == L && tl.p + 1 < c.n_chunks) {
    Common cn = c;
    cn.lb += region;
    stress_pause(cn, tl.p, tl.chain, 3);
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int k = 0; k < S; ++k)
        st_word(word_at<S, TW, NSLOT>(cn, tl.p, tl.chain, Op::HALO + k, q0 + v), c.tag, rg.h[k][L][v]);
  }
  if (tl.slice == TS - 1) {
#pragma unroll
    for (int k = 0; k < S; ++k)
#pragma unroll
      for (int v = 0; v < V; ++v) sh_last[k][tl.wave][q0 + v] = rg.h[k][L][v];
  }
  __syncthreads();
}

// waves per SIMD the fused kernel's registers must leave room for: four (two workgroups of 8 waves per CU)
// when the gate inputs parked in LDS leave room for two workgroups in the CU's 160 KB, else two (the
// fp32 GRU: 96 KB of inputs)
template <class Op>
struct FuseMinw {
  static constexpr int value = Op::UWORDS * Op::NW * WAVE * 4 <= 64 * 1024 ? 4 : 2;
};
// MASKED: the launch has lanes whose steps end at T (T not a multiple of the tile's steps); without it every
// lane takes the unmasked elements, as k_tile's full lanes do
template <class Op, bool MASKED, bool LOOP = false>   // LOOP: as for k_tile
__global__ __launch_bounds__(Op::NW * WAVE) __attribute__((amdgpu_waves_per_eu(FuseMinw<Op>::value)))
void k_fused(const typename Op::Args a, const FuseArgs f) {
  constexpr int S = Op::S, V = Op::V, L = Op::L, NW = Op::NW, TS = Op::TS;
  constexpr int TW = (WAVE / TS) * V;
  static_assert(Op::FUSABLE && !Op::REVERSE, "fused Newton pass");
  PR_TILE_SHM(Op);
  __shared__ float sh_last[S][NW][TW];   // each wave's state at its last step
  __shared__ uint32_t sh_u[Op::UWORDS][NW * WAVE];   // each lane's gate inputs (lane-minor: no bank conflicts)
  __shared__ float sh_pm[Op::G][4][TW];              // the tile's channel parameters (w, bias, sw, sb)

  if (Op::skip(a)) return;   // uniform, as in k_tile
  int m = f.m;
  if (f.redo) {
    m = Op::redo_count(a, f.m);
    if (m == 0) return;
  }
  while (true) {
    if (threadIdx.x == 0)
      sh_ticket = __hip_atomic_fetch_add(a.c.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if constexpr (LOOP) {
      if (sh_ticket >= static_cast<uint32_t>(a.c.n_chains) * static_cast<uint32_t>(a.c.n_chunks)) return;
    }
    Tile tl;
    tile_setup<NW, TS, L, V, false>(a.c, sh_ticket, tl);

    typename Op::Regs rg;
    if (!MASKED || tl.nvalid == L) Op::template load<false>(a, tl, rg);
    else Op::template load<true>(a, tl, rg);
    {
      // the gate inputs wait in LDS (each lane its own slots) and are read back at every iteration, the
      // first included: nothing derived from them stays live in registers across the scan's barriers
      uint32_t w[Op::UWORDS];
      Op::pack_u(rg, w);
#pragma unroll
      for (int q = 0; q < Op::UWORDS; ++q) sh_u[q][threadIdx.x] = w[q];
      if (tl.first_seg) {
        const int q0 = tl.qlane * V;
#pragma unroll
        for (int g = 0; g < Op::G; ++g)
#pragma unroll
          for (int v = 0; v < V; ++v) {
            sh_pm[g][0][q0 + v] = rg.pm.w[g][v];
            sh_pm[g][1][q0 + v] = rg.pm.bias[g][v];
            sh_pm[g][2][q0 + v] = rg.pm.sw[g][v];
            sh_pm[g][3][q0 + v] = rg.pm.sb[g][v];
          }
      }
    }
    __syncthreads();

    // every iteration but the last keeps the trajectory in registers; the last one stores it
    typename Op::Lane ln;
    float x[V][S];
    for (int j = 0; j + 1 < m; ++j) {
      Common c = a.c;
      c.lb += j * f.region;
      fused_inputs<Op>(tl, sh_pm, rg);
      if (j > 0) fused_enter<Op>(c, tl, sh_last, rg);
      // in a MASKED launch the masked elements serve every lane: on full lanes they equal the unmasked ones
      const float rmax = Op::template elements<MASKED, false>(tl, rg, ln, LdsU<Op>{sh_u});
      tile_scan<Op>(a, c, a.res_slot + j, tl, ln, rmax, sh, x);
      Op::template advance<MASKED>(tl, ln, x, rg);
      fused_leave<Op>(c, f.region, tl, sh_last, rg);
    }
    Common c = a.c;
    c.lb += (m - 1) * f.region;
    fused_inputs<Op>(tl, sh_pm, rg);
    if (m > 1) fused_enter<Op>(c, tl, sh_last, rg);
    const float rmax = Op::template elements<MASKED, false>(tl, rg, ln, LdsU<Op>{sh_u});
    tile_scan<Op>(a, c, a.res_slot + (m - 1), tl, ln, rmax, sh, x);
    // the stores' addressing from the ticket re-read after the loop, so the compiler cannot compute it early
    // and keep it in registers through every iteration
    Tile te;
    tile_setup<NW, TS, L, V, false>(a.c, sh_ticket, te);
    Op::finish(a, te, ln, x);
    if constexpr (!LOOP) return;
    __syncthreads();   // the tile's shared memory and ticket are free again
  }
}

// ------------------------------------------------------------------------------------------------
// auxiliary kernels
// ------------------------------------------------------------------------------------------------
// zero-fill (used instead of hipMemsetAsync so that the calls stay capturable)
__global__ void k_zero(uint4* p, int64_t n16) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// packed sequences: offsets cu[0 .. n-1] -> mask bit s for every offset 0 < s < T (the mask was
// zeroed by k_zero before; offsets outside that range mark nothing)
__global__ void k_segmask(const int32_t* cu, int64_t n, int64_t T, uint32_t* mask) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (j >= n) return;
  const int64_t s = cu[j];
  if (s > 0 && s < T) atomicOr(mask + (s >> 5), 1u << (s & 31));
}

// Parameter gradients from the per-tile partials [n_chunks][npar][B*D] in a fixed order (bitwise
// reproducible): stage 1 splits the B*n_chunks rows into kRedSlices contiguous slices and sums each
// slice per output (rows in ascending order within kRedRows interleaved groups, the groups in order);
// stage 2 sums the slices in order and writes d_w / d_bias.
constexpr int kRedCols = 64, kRedRows = 4, kRedSlices = 32, kRedUnroll = 8;
__global__ __launch_bounds__(kRedCols * kRedRows) void k_param_reduce1(const float* partial, int64_t n_chunks,
                                                                      int npar, int64_t B, int64_t D,
                                                                      float* slices) {
  __shared__ float sh[kRedRows][kRedCols];
  const int col = threadIdx.x % kRedCols, rg = threadIdx.x / kRedCols;
  const int64_t o = static_cast<int64_t>(blockIdx.x) * kRedCols + col;   // output index j*D + d
  const int64_t C = B * D, R = B * n_chunks, n_out = npar * D;
  const int64_t per = (R + kRedSlices - 1) / kRedSlices;
  const int64_t r0 = blockIdx.y * per, r1 = r0 + per < R ? r0 + per : R;
  float sum = 0.0f;
  if (o < n_out && r0 + rg < r1) {
    const int j = static_cast<int>(o / D);
    const int64_t d = o - j * D;
    // row r = b * n_chunks + ch, stepped kRedRows at a time without a division per row; kRedUnroll rows'
    // loads are issued before their sums (which still run in row order)
    int64_t b = (r0 + rg) / n_chunks, ch = r0 + rg - b * n_chunks;
    for (int64_t r = r0 + rg; r < r1; r += kRedRows * kRedUnroll) {
      float v[kRedUnroll];
#pragma unroll
      for (int u = 0; u < kRedUnroll; ++u) {
        v[u] = r + u * kRedRows < r1 ? partial[(ch * npar + j) * C + b * D + d] : 0.0f;
        ch += kRedRows;
        while (ch >= n_chunks) {
          ch -= n_chunks;
          ++b;
        }
      }
#pragma unroll
      for (int u = 0; u < kRedUnroll; ++u)
        if (r + u * kRedRows < r1) sum += v[u];
    }
  }
  sh[rg][col] = sum;
  __syncthreads();
  if (rg == 0 && o < n_out) {
    float t = 0.0f;
#pragma unroll
    for (int i = 0; i < kRedRows; ++i) t += sh[i][col];
    slices[blockIdx.y * n_out + o] = t;
  }
}

__global__ __launch_bounds__(256) void k_param_reduce2(const float* slices, int npar, int64_t D, float* d_w,
                                                      float* d_bias, int G) {
  const int64_t o = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x, n_out = npar * D;
  if (o >= n_out) return;
  float t = 0.0f;
  for (int i = 0; i < kRedSlices; ++i) t += slices[i * n_out + o];
  const int j = static_cast<int>(o / D);
  const int64_t d = o - j * D;
  if (j < G) {
    if (d_w) d_w[j * D + d] = t;
  } else {
    if (d_bias) d_bias[(j - G) * D + d] = t;
  }
}

// max |h_t - f(h_{t-1}, x_t)| of a trajectory (the optional final-residual pass); one thread per
// V channels x L steps, read-only
template <int CELL, int DT, int V, int L>
__global__ __launch_bounds__(256) void k_residual(const void* p0, const void* p1, const void* p2,
                                                  const void* p3, const float* w, const float* bias,
                                                  const float* s0, const float* h, int64_t B, int64_t T,
                                                  int64_t D, const uint32_t* seg, uint32_t* out) {
  constexpr int S = CellInfo<CELL>::S, G = CellInfo<CELL>::G;
  const void* pre[4] = {p0, p1, p2, p3};
  const int64_t C = B * D, N = B * T * D;
  const int64_t n_col = (C + V - 1) / V;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t col = gid % n_col, chunk = gid / n_col;
  float m = 0.0f;
  if (chunk * L < T && col * V < C) {
    const int64_t ch0 = col * V, b = ch0 / D, d0 = ch0 - b * D;
    Params<G, V> pm;
    if constexpr (CELL != CELL_LINEAR) load_params<CELL, G, V>(w, bias, D, d0, pm);
    for (int i = 0; i < L; ++i) {
      const int64_t t = chunk * L + i;
      if (t >= T) break;
      const int64_t idx = (b * T + t) * D + d0;
      float prev[S][V], cur[S][V], u[G][V];
      const bool rs = seg && ((seg[t >> 5] >> (t & 31)) & 1u);   // a packed sequence begins at t
#pragma unroll
      for (int k = 0; k < S; ++k) {
        if (rs) {
#pragma unroll
          for (int v = 0; v < V; ++v) prev[k][v] = 0.0f;
        } else if (t == 0) {
          if (s0) ldv<V, DT_F32>(s0, (k * B + b) * D + d0, prev[k]);
          else
#pragma unroll
            for (int v = 0; v < V; ++v) prev[k][v] = 0.0f;
        } else {
          ldv<V, DT_F32>(h, k * N + idx - D, prev[k]);
        }
        ldv<V, DT_F32>(h, k * N + idx, cur[k]);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) ldv<V, DT>(pre[g], idx, u[g]);
#pragma unroll
      for (int v = 0; v < V; ++v) {
        if constexpr (CELL == CELL_LINEAR) {
          m = nanmax(m, fabsf(cur[0][v] - fmaf(u[0][v], prev[0][v], u[1][v])));
        } else if constexpr (CELL == CELL_GRU) {
          const GruOut q = gru_eval(pm, v, u[0][v], u[1][v], u[2][v], prev[0][v]);
          m = nanmax(m, fabsf(cur[0][v] - q.f));
        } else if constexpr (CELL == CELL_LSTM) {
          const LstmPart q = lstm_eval(pm, v, u[0][v], u[1][v], u[2][v], u[3][v], prev[0][v], prev[1][v]);
          m = nanmax(m, fabsf(cur[0][v] - q.c2));
          m = nanmax(m, fabsf(cur[1][v] - q.h2));
        } else {
          const SlstmPart q = slstm_eval(pm, v, u[0][v], u[1][v], u[2][v], u[3][v], prev[0][v], prev[1][v],
                                         prev[2][v], prev[3][v]);
#pragma unroll
          for (int k = 0; k < 4; ++k) m = nanmax(m, fabsf(cur[k][v] - q.s2[k]));
        }
      }
    }
  }
  m = wave_nanmax(m);
  if ((threadIdx.x % WAVE) == 0) atomicMax(out, __float_as_uint(m));
}

#include "head_gru_dev.inc"

}  // namespace pr

// ================================================================================================
// host side
// ================================================================================================
namespace {

using namespace pr;

std::atomic<uint32_t> g_tag{0};
uint32_t next_tag() {
  uint32_t t;
  do {
    t = g_tag.fetch_add(1, std::memory_order_relaxed) + 1;
  } while (t == 0);
  return t;
}

int state_size(int cell) { return cell == CELL_SLSTM ? 4 : (cell == CELL_LSTM ? 2 : 1); }
int gate_count(int cell) {
  return (cell == CELL_LSTM || cell == CELL_SLSTM) ? 4 : ((cell == CELL_GRU || cell == CELL_HEAD_GRU) ? 3 : 2);
}

// workspace: [header 4 KiB: tickets, residual slots][packed-sequence mask][look-back words]
// [VJP partials]; the mask is (T >> 5) + 2 words (read two at a time by seg_bits)
constexpr size_t kHeader = 4096;
constexpr size_t kResOffset = 2048;  // residual slots (uint32 float bits) inside the header
constexpr int kRedoTicket = PARARNN_MAX_ITERS + 1;   // ticket slot of a fused pass's re-run launch

// bound on the number of packed sequences (offsets are int32 steps)
constexpr int64_t kMaxSeqs = INT32_MAX - 1;

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
size_t seg_bytes(int64_t T) { return align256(static_cast<size_t>((T >> 5) + 2) * sizeof(uint32_t)); }
size_t lb_offset(int64_t T) { return kHeader + seg_bytes(T); }
uint32_t* seg_mask(void* ws) { return reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + kHeader); }

struct Geo {
  int V, L, NW, S, nslot;
  int64_t TW, CT, n_chains, n_chunks;
  size_t lb_bytes() const {
    return static_cast<size_t>(n_chunks) * n_chains * nslot * TW * sizeof(uint64_t);
  }
};

Geo make_geo(int S, int nslot, int V, int L, int NW, int TS, int64_t B, int64_t T, int64_t D) {
  Geo g;
  g.V = V; g.L = L; g.NW = NW; g.S = S; g.nslot = nslot;
  g.TW = (WAVE / TS) * V;
  g.CT = static_cast<int64_t>(NW) * TS * L;
  const int64_t C = B * D;
  g.n_chains = (C + g.TW - 1) / g.TW;
  g.n_chunks = (T + g.CT - 1) / g.CT;
  return g;
}

// tile configurations (V channels per lane, L steps per lane, NW waves per workgroup, and the
// minimum waves per SIMD the register allocation must leave room for); the same values instantiate
// the kernels and size the workspaces.  The PR_* macros exist for tuning builds.
#ifndef PR_GRU_CFG
#define PR_GRU_CFG 1, 16, 8, 4, 2
#endif
#ifndef PR_LSTM_CFG
#define PR_LSTM_CFG 1, 8, 8, 4, 2
#endif
#ifndef PR_SCAN1_CFG
#define PR_SCAN1_CFG 1, 16, 16, 4, 1
#endif
#ifndef PR_SCAN2_CFG
#define PR_SCAN2_CFG 1, 8, 16, 4, 1
#endif
#ifndef PR_VJP_GRU_CFG
#define PR_VJP_GRU_CFG 1, 8, 16, 4, 1
#endif
#ifndef PR_SLSTM_CFG
#define PR_SLSTM_CFG 1, 8, 4, 2, 2
#endif
#ifndef PR_VJP_SLSTM_CFG
#define PR_VJP_SLSTM_CFG 1, 12, 4, 2, 2
#endif
#ifndef PR_VJP_LSTM_CFG
#define PR_VJP_LSTM_CFG 1, 4, 16, 4, 1
#endif
template <int V_, int L_, int NW_, int MINW_, int TS_>
struct TileCfg { static constexpr int V = V_, L = L_, NW = NW_, MINW = MINW_, TS = TS_; };
template <int CELL> struct NewtonCfg : TileCfg<PR_GRU_CFG> {};
template <> struct NewtonCfg<CELL_LSTM> : TileCfg<PR_LSTM_CFG> {};
template <> struct NewtonCfg<CELL_SLSTM> : TileCfg<PR_SLSTM_CFG> {};
template <int S> struct ScanCfg : TileCfg<PR_SCAN1_CFG> {};
template <> struct ScanCfg<2> : TileCfg<PR_SCAN2_CFG> {};
template <int CELL> struct VjpCfg : TileCfg<PR_VJP_GRU_CFG> {};
template <> struct VjpCfg<CELL_LSTM> : TileCfg<PR_VJP_LSTM_CFG> {};
template <> struct VjpCfg<CELL_SLSTM> : TileCfg<PR_VJP_SLSTM_CFG> {};
template <int CELL, int DT, class C, bool SEG>
struct VjpOpOf { using type = VjpOp<CELL, DT, C::V, C::L, C::NW, C::MINW, C::TS, SEG>; };
template <int DT, class C, bool SEG>
struct VjpOpOf<CELL_SLSTM, DT, C, SEG> { using type = SlstmVjpOp<DT, C::V, C::L, C::NW, C::MINW, C::TS, SEG>; };

Common make_common(void* ws, const Geo& g, int64_t B, int64_t T, int64_t D, int ticket_slot) {
  Common c;
  char* base = static_cast<char*>(ws);
  c.lb = reinterpret_cast<uint64_t*>(base + lb_offset(T));
  c.seg = seg_mask(ws);
  c.ticket = reinterpret_cast<uint32_t*>(base) + ticket_slot;
  c.tag = 0;
  c.n_chains = static_cast<int32_t>(g.n_chains);
  c.n_chunks = g.n_chunks;
  c.T = T; c.D = D; c.C = B * D; c.N = B * T * D;
  // largest lane offset from its wave's base element: a lane is at most ceil(TW / D) rows further
  // (the row length T*D each), TS*L steps, and less than TW + D channels away; in fp32 bytes
  const int64_t rows = (g.TW + D - 1) / D;
  const double max_off = (static_cast<double>(rows) * T * D + static_cast<double>(g.CT) * D + g.TW + D) * 4.0;
  c.off32 = max_off < 4294967296.0 ? 1 : 0;
  return c;
}

pararnn_status launch_zero(void* p, size_t bytes, hipStream_t st) {
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  if (n16 == 0) return PARARNN_OK;
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_zero, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, static_cast<uint4*>(p), n16);
  return hipGetLastError() == hipSuccess ? PARARNN_OK : PARARNN_ERR_HIP;
}

// clear the header, the mask and the look-back words; then mark the packed-sequence starts
pararnn_status prepare_ws(void* ws, int64_t T, size_t lb_bytes, const int32_t* cu, int64_t n_seqs, hipStream_t st) {
  pararnn_status rc = launch_zero(ws, lb_offset(T) + align256(lb_bytes), st);
  if (rc || !cu) return rc;
  const int64_t n = n_seqs + 1;
  hipLaunchKernelGGL(k_segmask, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, cu, n, T,
                     seg_mask(ws));
  return hipGetLastError() == hipSuccess ? PARARNN_OK : PARARNN_ERR_HIP;
}

template <class Op>
pararnn_status launch_tile(const typename Op::Args& a, const Geo& g, hipStream_t st) {
  const int64_t tiles = g.n_chains * g.n_chunks;
  if (tiles <= 0) return PARARNN_OK;
  hipLaunchKernelGGL(k_tile<Op>, dim3(static_cast<unsigned>(tiles)), dim3(Op::NW * WAVE), 0, st, a);
  return hipGetLastError() == hipSuccess ? PARARNN_OK : PARARNN_ERR_HIP;
}

// workgroups of `kernel` (blocks of `threads`) the current device holds at once, cached per device in
// `cache`; 0 when HIP cannot tell
constexpr int kMaxDevices = 256;
template <class F>
int64_t resident_grid(F kernel, int threads, std::atomic<int>* cache) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    v = per_cu * cus;
    if (v <= 0) return 0;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// k_tile<Op, LOOP = true> on a grid of what is resident (at most one workgroup per tile)
template <class Op>
pararnn_status launch_tile_loop(const typename Op::Args& a, const Geo& g, hipStream_t st) {
  const int64_t tiles = g.n_chains * g.n_chunks;
  if (tiles <= 0) return PARARNN_OK;
  static std::atomic<int> cache[kMaxDevices];
  int64_t grid = resident_grid(k_tile<Op, true>, Op::NW * WAVE, cache);
  if (grid <= 0 || grid > tiles) grid = tiles;
  hipLaunchKernelGGL((k_tile<Op, true>), dim3(static_cast<unsigned>(grid)), dim3(Op::NW * WAVE), 0, st, a);
  return hipGetLastError() == hipSuccess ? PARARNN_OK : PARARNN_ERR_HIP;
}

bool grid_ok(const Geo& g) {
  const int64_t tiles = g.n_chains * g.n_chunks;
  return tiles < (static_cast<int64_t>(1) << 31);
}

// ---------------- validation ----------------
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// nonnegative B, T, D (B and D at most 2^40) whose element count, times the 4 planes of the largest cell and
// 4 bytes an element, fits int64 (every product is tested by division before it is formed)
bool sizes_fit(int64_t B, int64_t T, int64_t D) {
  if (B < 0 || T < 0 || D < 0) return false;
  if (B > (int64_t(1) << 40) || D > (int64_t(1) << 40)) return false;
  if (B == 0 || T == 0 || D == 0) return true;
  const int64_t lim = INT64_MAX / 16;
  if (B > lim / D) return false;
  return T <= lim / (B * D);
}

pararnn_status check_problem(const pararnn_problem* pb) {
  if (!pb) return PARARNN_ERR_INVALID_ARG;
  if (pb->cell < CELL_LINEAR || pb->cell > CELL_HEAD_GRU) return PARARNN_ERR_INVALID_ARG;
  if (pb->pre_dtype != PARARNN_F32 && pb->pre_dtype != PARARNN_BF16) return PARARNN_ERR_INVALID_ARG;
  if (pb->B < 0 || pb->T < 0 || pb->D < 0) return PARARNN_ERR_INVALID_ARG;
  if (!sizes_fit(pb->B, pb->T, pb->D)) return PARARNN_ERR_INVALID_ARG;
  if (pb->cell == CELL_HEAD_GRU) {
    if (pb->head_size < 1 || (pb->D > 0 && pb->D % pb->head_size != 0)) return PARARNN_ERR_INVALID_ARG;
    if (pb->head_size != 16 && pb->head_size != 32 && pb->head_size != 64) return PARARNN_ERR_UNSUPPORTED;
  }
  const int64_t N = pb->B * pb->T * pb->D;
  if (N == 0) return PARARNN_OK;
  if (pb->D % 2 != 0) return PARARNN_ERR_UNSUPPORTED;
  const int G = gate_count(pb->cell);
  for (int g = 0; g < G; ++g)
    if (!pb->pre[g] || !aligned(pb->pre[g], 8)) return PARARNN_ERR_INVALID_ARG;
  if (pb->cell != CELL_LINEAR && (!pb->w || !pb->bias || !aligned(pb->w, 8) || !aligned(pb->bias, 8)))
    return PARARNN_ERR_INVALID_ARG;
  if (pb->s0 && !aligned(pb->s0, 8)) return PARARNN_ERR_INVALID_ARG;
  if (pb->cu_seqlens && (!aligned(pb->cu_seqlens, 4) || pb->n_seqs < 0 || pb->n_seqs > kMaxSeqs))
    return PARARNN_ERR_INVALID_ARG;
  return PARARNN_OK;
}

int64_t problem_N(const pararnn_problem* pb) { return pb->B * pb->T * pb->D; }

// ---------------- Newton ----------------
template <int CELL, int DT, bool SEG>
struct NewtonKernel {
  using C = NewtonCfg<CELL>;
  using Op = NewtonOp<CELL, DT, C::V, C::L, C::NW, C::MINW, C::TS, SEG>;
  static Geo geo(const pararnn_problem* pb) {
    return make_geo(Op::S, Op::NSLOT, C::V, C::L, C::NW, C::TS, pb->B, pb->T, pb->D);
  }
  // `regions` look-back word regions: one per iteration of the longest fused pass (1 without fusion)
  static size_t ws(const pararnn_problem* pb, int regions) {
    return lb_offset(pb->T) + static_cast<size_t>(regions) * align256(geo(pb).lb_bytes());
  }
  static pararnn_status prepare(const pararnn_problem* pb, void* ws, int regions, hipStream_t st) {
    const Geo g = geo(pb);
    if (!grid_ok(g)) return PARARNN_ERR_UNSUPPORTED;
    return prepare_ws(ws, pb->T, static_cast<size_t>(regions) * align256(g.lb_bytes()), pb->cu_seqlens, pb->n_seqs,
                      st);
  }
  static typename Op::Args args(const pararnn_problem* pb, const pararnn_newton_opts* op, int k, float* s_out,
                                void* ws, const Geo& g, int ticket_slot) {
    uint32_t* res = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + kResOffset);
    typename Op::Args a;
    a.c = make_common(ws, g, pb->B, pb->T, pb->D, ticket_slot);
    a.c.tag = next_tag();
    for (int i = 0; i < 4; ++i) a.pre[i] = pb->pre[i];
    a.w = pb->w;
    a.bias = pb->bias;
    a.s0 = pb->s0;
    a.h_in = (k == 0) ? op->init_guess : s_out;
    a.h_out = s_out;
    a.warm = op->init_mode == PARARNN_INIT_WARM;
    a.picard = k < op->picard_iters ? 1 : 0;
    a.res_slot = res + k;
    a.res_hist = res;
    a.k = k;
    a.tol = op->tol;
    a.B = pb->B;
    return a;
  }
  static pararnn_status iterate(const pararnn_problem* pb, const pararnn_newton_opts* op, int k, float* s_out,
                                void* ws, hipStream_t st) {
    const Geo g = geo(pb);
    if (!grid_ok(g)) return PARARNN_ERR_UNSUPPORTED;
    return launch_tile<Op>(args(pb, op, k, s_out, ws, g, k), g, st);
  }
  // iteration k after a speculative fused pass (past the first single launch): the same work on a grid of
  // what is resident, since the launch mostly finds the solve stopped
  static pararnn_status iterate_tail(const pararnn_problem* pb, const pararnn_newton_opts* op, int k, float* s_out,
                                     void* ws, hipStream_t st) {
    const Geo g = geo(pb);
    if (!grid_ok(g)) return PARARNN_ERR_UNSUPPORTED;
    return launch_tile_loop<Op>(args(pb, op, k, s_out, ws, g, k), g, st);
  }
  // iterations k .. k+m-1 in one launch of k_fused (redo: the re-run launch of a speculative pass, on a
  // grid of what is resident, since it mostly finds nothing to re-run)
  static pararnn_status fused(const pararnn_problem* pb, const pararnn_newton_opts* op, int k, int m, bool redo,
                              float* s_out, void* ws, hipStream_t st) {
    if constexpr (!Op::FUSABLE) {
      return PARARNN_ERR_UNSUPPORTED;
    } else {
      const Geo g = geo(pb);
      if (!grid_ok(g)) return PARARNN_ERR_UNSUPPORTED;
      const typename Op::Args a = args(pb, op, k, s_out, ws, g, redo ? kRedoTicket : k);
      FuseArgs f;
      f.m = m;
      f.redo = redo ? 1 : 0;
      f.region = static_cast<int64_t>(align256(g.lb_bytes()) / sizeof(uint64_t));
      const int64_t tiles = g.n_chains * g.n_chunks;
      const dim3 block(Op::NW * WAVE);
      const bool masked = pb->T % g.CT != 0;
      if (redo) {
        static std::atomic<int> cache[2][kMaxDevices];
        int64_t grid = masked ? resident_grid(k_fused<Op, true, true>, Op::NW * WAVE, cache[1])
                              : resident_grid(k_fused<Op, false, true>, Op::NW * WAVE, cache[0]);
        if (grid <= 0 || grid > tiles) grid = tiles;
        if (masked) hipLaunchKernelGGL((k_fused<Op, true, true>), dim3(static_cast<unsigned>(grid)), block, 0, st, a, f);
        else hipLaunchKernelGGL((k_fused<Op, false, true>), dim3(static_cast<unsigned>(grid)), block, 0, st, a, f);
      } else if (masked) {
        hipLaunchKernelGGL((k_fused<Op, true>), dim3(static_cast<unsigned>(tiles)), block, 0, st, a, f);
      } else {
        hipLaunchKernelGGL((k_fused<Op, false>), dim3(static_cast<unsigned>(tiles)), block, 0, st, a, f);
      }
      return hipGetLastError() == hipSuccess ? PARARNN_OK : PARARNN_ERR_HIP;
    }
  }
  static pararnn_status final_residual(const pararnn_problem* pb, const float* s_out, void* ws, hipStream_t st) {
    uint32_t* res = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + kResOffset);
    constexpr int RV = 2, RL = 16;
    const int64_t C = pb->B * pb->D;
    const int64_t threads = ((C + RV - 1) / RV) * ((pb->T + RL - 1) / RL);
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL((k_residual<CELL, DT, RV, RL>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                       pb->pre[0], pb->pre[1], pb->pre[2], pb->pre[3], pb->w, pb->bias, pb->s0, s_out, pb->B,
                       pb->T, pb->D, SEG ? seg_mask(ws) : nullptr, res + PARARNN_MAX_ITERS);
    return hipGetLastError() == hipSuccess ? PARARNN_OK : PARARNN_ERR_HIP;
  }
};

// Tolerance mode, cells without a fused pass (the sLSTM): the Newton iterations from this many after the
// Picard sweeps on run on a grid of what is resident, as the launches after a speculative fused pass do.  Once
// the solve has stopped such a launch exits in a few us, where one workgroup per tile costs up to ~160 us
// (B=8, T=65536, D=256); while it still works it is ~15% slower (the looping kernel spills).  The sLSTM
// workloads stop after 8-17 Newton iterations.  The launch shape leaves every result the same bit for bit.
#ifndef PR_TAIL_FROM
#define PR_TAIL_FROM 12
#endif
struct NewtonEntry {
  size_t (*ws)(const pararnn_problem*, int);
  pararnn_status (*prepare)(const pararnn_problem*, void*, int, hipStream_t);
  pararnn_status (*iterate)(const pararnn_problem*, const pararnn_newton_opts*, int, float*, void*, hipStream_t);
  pararnn_status (*final_residual)(const pararnn_problem*, const float*, void*, hipStream_t);
  // NULL for cells without a fused pass
  pararnn_status (*fused)(const pararnn_problem*, const pararnn_newton_opts*, int, int, bool, float*, void*,
                          hipStream_t);
  // the single launches that usually find the solve stopped: after the first one that follows a speculative
  // fused pass, or (cells without a fused pass) late tolerance-mode iterations
  pararnn_status (*iterate_tail)(const pararnn_problem*, const pararnn_newton_opts*, int, float*, void*,
                                 hipStream_t);
};

template <int CELL, int DT, bool SEG>
NewtonEntry newton_entry() {
  using K = NewtonKernel<CELL, DT, SEG>;
  if constexpr (K::Op::FUSABLE) return {K::ws, K::prepare, K::iterate, K::final_residual, K::fused, K::iterate_tail};
  else return {K::ws, K::prepare, K::iterate, K::final_residual, nullptr, K::iterate_tail};
}

template <int CELL, int DT>
NewtonEntry newton_entry_seg(bool seg) { return seg ? newton_entry<CELL, DT, true>() : newton_entry<CELL, DT, false>(); }

template <int CELL>
NewtonEntry newton_entry_dt(int dt, bool seg) {
  return dt == DT_BF16 ? newton_entry_seg<CELL, DT_BF16>(seg) : newton_entry_seg<CELL, DT_F32>(seg);
}

NewtonEntry pick_head_newton(const pararnn_problem* pb);

NewtonEntry pick_newton(const pararnn_problem* pb) {
  if (pb->cell == CELL_HEAD_GRU) return pick_head_newton(pb);
  const bool seg = pb->cu_seqlens != nullptr;
  if (pb->cell == CELL_GRU) return newton_entry_dt<CELL_GRU>(pb->pre_dtype, seg);
  if (pb->cell == CELL_LSTM) return newton_entry_dt<CELL_LSTM>(pb->pre_dtype, seg);
  if (pb->cell == CELL_SLSTM) return newton_entry_dt<CELL_SLSTM>(pb->pre_dtype, seg);
  return newton_entry_dt<CELL_LINEAR>(pb->pre_dtype, seg);
}

// ---------------- linear scan ----------------
template <int S, int DT, bool REV, bool SEG>
struct ScanKernel {
  using C = ScanCfg<S>;
  using Op = LinearOp<S, DT, REV, C::V, C::L, C::NW, C::MINW, C::TS, SEG>;
  static Geo geo(int64_t B, int64_t T, int64_t D) { return make_geo(S, Op::NSLOT, C::V, C::L, C::NW, C::TS, B, T, D); }
  static size_t ws(int64_t B, int64_t T, int64_t D) { return lb_offset(T) + align256(geo(B, T, D).lb_bytes()); }
  static pararnn_status run(int64_t B, int64_t T, int64_t D, const void* a_, const void* b_, const float* s0,
                            const int32_t* cu, int64_t n_seqs, float* out, void* ws, hipStream_t st) {
    const Geo g = geo(B, T, D);
    if (!grid_ok(g)) return PARARNN_ERR_UNSUPPORTED;
    pararnn_status rc = prepare_ws(ws, T, g.lb_bytes(), cu, n_seqs, st);
    if (rc) return rc;
    typename Op::Args a;
    a.c = make_common(ws, g, B, T, D, 0);
    a.c.tag = next_tag();
    a.a = a_;
    a.b = b_;
    a.s0 = s0;
    a.out = out;
    a.B = B;
    a.res_slot = nullptr;
    return launch_tile<Op>(a, g, st);
  }
};

struct ScanEntry {
  size_t (*ws)(int64_t, int64_t, int64_t);
  pararnn_status (*run)(int64_t, int64_t, int64_t, const void*, const void*, const float*, const int32_t*, int64_t,
                        float*, void*, hipStream_t);
};

template <int S, int DT, bool REV, bool SEG>
ScanEntry scan_entry() { return {ScanKernel<S, DT, REV, SEG>::ws, ScanKernel<S, DT, REV, SEG>::run}; }

template <int S, int DT, bool REV>
ScanEntry pick_scan_seg(bool seg) { return seg ? scan_entry<S, DT, REV, true>() : scan_entry<S, DT, REV, false>(); }

template <int S, int DT>
ScanEntry pick_scan_dir(int rev, bool seg) {
  return rev ? pick_scan_seg<S, DT, true>(seg) : pick_scan_seg<S, DT, false>(seg);
}

ScanEntry pick_scan(int S, int dt, int rev, bool seg) {
  if (S == 1) return dt == DT_BF16 ? pick_scan_dir<1, DT_BF16>(rev, seg) : pick_scan_dir<1, DT_F32>(rev, seg);
  return dt == DT_BF16 ? pick_scan_dir<2, DT_BF16>(rev, seg) : pick_scan_dir<2, DT_F32>(rev, seg);
}

// ---------------- VJP ----------------
template <int CELL, int DT, bool SEG>
struct VjpKernel {
  using C = VjpCfg<CELL>;
  using Op = typename VjpOpOf<CELL, DT, C, SEG>::type;
  static Geo geo(const pararnn_problem* pb) {
    return make_geo(Op::S, Op::NSLOT, C::V, C::L, C::NW, C::TS, pb->B, pb->T, pb->D);
  }
  static size_t part_bytes(const Geo& g, const pararnn_problem* pb) {
    return static_cast<size_t>(g.n_chunks) * Op::NPAR * pb->B * pb->D * sizeof(float);
  }
  static size_t slice_bytes(const pararnn_problem* pb) {
    return static_cast<size_t>(kRedSlices) * Op::NPAR * pb->D * sizeof(float);
  }
  static size_t ws(const pararnn_problem* pb) {
    const Geo g = geo(pb);
    return lb_offset(pb->T) + align256(g.lb_bytes()) + align256(part_bytes(g, pb)) + align256(slice_bytes(pb));
  }
  static pararnn_status run(const pararnn_problem* pb, const float* s, const float* gr, float* d_pre, float* d_w,
                            float* d_bias, float* d_s0, float* lam, void* ws, hipStream_t st) {
    const Geo g = geo(pb);
    if (!grid_ok(g)) return PARARNN_ERR_UNSUPPORTED;
    const size_t lbb = align256(g.lb_bytes());
    pararnn_status rc = prepare_ws(ws, pb->T, g.lb_bytes(), pb->cu_seqlens, pb->n_seqs, st);
    if (rc) return rc;
    typename Op::Args a;
    a.c = make_common(ws, g, pb->B, pb->T, pb->D, 0);
    a.c.tag = next_tag();
    for (int i = 0; i < 4; ++i) a.pre[i] = pb->pre[i];
    a.w = pb->w;
    a.bias = pb->bias;
    a.s0 = pb->s0;
    a.s = s;
    a.g = gr;
    a.d_pre = d_pre;
    a.lambda_out = lam;
    a.d_s0 = d_s0;
    a.partial = reinterpret_cast<float*>(static_cast<char*>(ws) + lb_offset(pb->T) + lbb);
    a.B = pb->B;
    a.res_slot = nullptr;
    rc = launch_tile<Op>(a, g, st);
    if (rc) return rc;
    if constexpr (Op::NPAR > 0) {
      if (d_w || d_bias) {
        const int64_t n = Op::NPAR * pb->D;
        float* slices = reinterpret_cast<float*>(reinterpret_cast<char*>(a.partial) + align256(part_bytes(g, pb)));
        hipLaunchKernelGGL(k_param_reduce1, dim3(static_cast<unsigned>((n + kRedCols - 1) / kRedCols), kRedSlices),
                           dim3(kRedCols * kRedRows), 0, st, a.partial, g.n_chunks, Op::NPAR, pb->B, pb->D, slices);
        if (hipGetLastError() != hipSuccess) return PARARNN_ERR_HIP;
        hipLaunchKernelGGL(k_param_reduce2, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, slices,
                           Op::NPAR, pb->D, d_w, d_bias, Op::G);
        if (hipGetLastError() != hipSuccess) return PARARNN_ERR_HIP;
      }
    }
    return PARARNN_OK;
  }
};

struct VjpEntry {
  size_t (*ws)(const pararnn_problem*);
  pararnn_status (*run)(const pararnn_problem*, const float*, const float*, float*, float*, float*, float*, float*,
                        void*, hipStream_t);
};

template <int CELL, int DT, bool SEG>
VjpEntry vjp_entry() { return {VjpKernel<CELL, DT, SEG>::ws, VjpKernel<CELL, DT, SEG>::run}; }

template <int CELL, int DT>
VjpEntry vjp_entry_seg(bool seg) { return seg ? vjp_entry<CELL, DT, true>() : vjp_entry<CELL, DT, false>(); }

template <int CELL>
VjpEntry vjp_entry_dt(int dt, bool seg) {
  return dt == DT_BF16 ? vjp_entry_seg<CELL, DT_BF16>(seg) : vjp_entry_seg<CELL, DT_F32>(seg);
}

VjpEntry pick_head_vjp(const pararnn_problem* pb);

VjpEntry pick_vjp(const pararnn_problem* pb) {
  if (pb->cell == CELL_HEAD_GRU) return pick_head_vjp(pb);
  const bool seg = pb->cu_seqlens != nullptr;
  if (pb->cell == CELL_GRU) return vjp_entry_dt<CELL_GRU>(pb->pre_dtype, seg);
  if (pb->cell == CELL_LSTM) return vjp_entry_dt<CELL_LSTM>(pb->pre_dtype, seg);
  if (pb->cell == CELL_SLSTM) return vjp_entry_dt<CELL_SLSTM>(pb->pre_dtype, seg);
  return vjp_entry_dt<CELL_LINEAR>(pb->pre_dtype, seg);
}

#include "head_gru_host.inc"

}  // namespace

// ================================================================================================
// the allocation-free solve's workspace: one static device array, PARARNN_NOALLOC_SCRATCH_BYTES long,
// that every GPU the library runs on holds until the process ends.  Host code never passes the array's
// name to a kernel (in host code it is a host-side stand-in); it takes each device's own address of it
// once, with that device current, and uses that address.
// ================================================================================================
static __device__ __align__(256) unsigned char scratch[PARARNN_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // per device: the address of its copy of scratch (null until looked up)

pararnn_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PARARNN_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PARARNN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PARARNN_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PARARNN_OK;
}
}  // namespace

// ================================================================================================
// C ABI
// ================================================================================================
extern "C" {

int pararnn_abi_version(void) { return PARARNN_ABI_VERSION; }

const char* pararnn_status_string(int s) {
  switch (s) {
    case PARARNN_OK: return "ok";
    case PARARNN_ERR_INVALID_ARG: return "invalid argument";
    case PARARNN_ERR_UNSUPPORTED: return "unsupported configuration";
    case PARARNN_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case PARARNN_ERR_HIP: return "HIP runtime error";
    case PARARNN_ERR_DIVERGED: return "Newton diverged (non-finite residual, or the budget ended above the starting residual)";
    default: return "unknown status";
  }
}


namespace {
// common validation of the Newton entry points; `need_out` checks s_out as well
// Newton budget K*(T): the smallest iteration count whose iterate agreed with the sequential unroll
// to 1e-4 (max abs) on the seeded synthetic inputs of the benchmark workloads (B = 1, D = 1024; GRU
// with bf16 gate inputs, LSTM fp32), per first iterate, measured on a grid of lengths with the fp64
// oracle -- K*(T) as the pararnn-torch README defines it ("Method") and measures it in its
// long-context campaign ("Benchmarks").  A
// length between grid points takes the next larger point's budget; beyond the grid, one more.
// With each entry, the iteration count tolerance mode reached on the same inputs (the first k with R_k < tol,
// plus one) at tol = 1e-4, 1e-5 and 1e-6: the length of the speculative fused launch (fuse_len).
struct KStarRow { int32_t cell, init; int64_t T; int32_t k; int32_t stop[3]; };
constexpr KStarRow kKStar[] = {
    {CELL_GRU, PARARNN_INIT_ZERO, 1024, 3, {4, 5, 5}},
    {CELL_GRU, PARARNN_INIT_WARM, 1024, 3, {4, 4, 5}},
    {CELL_GRU, PARARNN_INIT_ZERO, 4096, 3, {4, 5, 5}},
    {CELL_GRU, PARARNN_INIT_WARM, 4096, 3, {4, 4, 5}},
    {CELL_GRU, PARARNN_INIT_ZERO, 16384, 3, {4, 5, 5}},
    {CELL_GRU, PARARNN_INIT_WARM, 16384, 3, {4, 4, 4}},
    {CELL_GRU, PARARNN_INIT_ZERO, 65536, 3, {4, 5, 5}},
    {CELL_GRU, PARARNN_INIT_WARM, 65536, 3, {4, 4, 5}},
    {CELL_GRU, PARARNN_INIT_ZERO, 131072, 3, {4, 5, 5}},
    {CELL_GRU, PARARNN_INIT_WARM, 131072, 3, {4, 4, 5}},
    {CELL_LSTM, PARARNN_INIT_ZERO, 1024, 4, {5, 5, 5}},
    {CELL_LSTM, PARARNN_INIT_WARM, 1024, 4, {5, 5, 5}},
    {CELL_LSTM, PARARNN_INIT_ZERO, 4096, 4, {5, 5, 5}},
    {CELL_LSTM, PARARNN_INIT_WARM, 4096, 4, {5, 5, 5}},
    {CELL_LSTM, PARARNN_INIT_ZERO, 16384, 4, {5, 5, 6}},
    {CELL_LSTM, PARARNN_INIT_WARM, 16384, 4, {5, 5, 5}},
    {CELL_LSTM, PARARNN_INIT_ZERO, 65536, 4, {5, 6, 6}},
    {CELL_LSTM, PARARNN_INIT_WARM, 65536, 4, {5, 5, 6}},
    {CELL_LSTM, PARARNN_INIT_ZERO, 131072, 4, {5, 5, 6}},
    {CELL_LSTM, PARARNN_INIT_WARM, 131072, 4, {5, 5, 5}},
};

int auto_iters(int cell, int init, int64_t T) {
  if (cell == CELL_LINEAR) return 1;  // one scan is exact
  int last = 0;
  for (const KStarRow& r : kKStar) {
    if (r.cell != cell || r.init != init) continue;
    if (T <= r.T) return r.k;
    last = r.k;
  }
  return last + 1;
}

// the tolerance-mode iteration count measured with K*(T), at the smallest of the table's tolerances (1e-4,
// 1e-5, 1e-6) at or above tol (a count no larger than tol's own on those inputs); beyond the grid, one more
int stop_iters(int cell, int init, int64_t T, float tol) {
  if (cell == CELL_LINEAR) return 1;
  const int col = tol > 1e-5f ? 0 : (tol > 1e-6f ? 1 : 2);
  int last = 0;
  for (const KStarRow& r : kKStar) {
    if (r.cell != cell || r.init != init) continue;
    if (T <= r.T) return r.stop[col];
    last = r.stop[col];
  }
  return last + 1;
}

// the budget a solve runs: max_iters, or K*(T) when max_iters is 0 (a caller-supplied first
// iterate counts as the zero start: nothing is known about its quality)
int budget(const pararnn_problem* pb, const pararnn_newton_opts* op) {
  if (op->max_iters > 0) return op->max_iters;
  return auto_iters(pb->cell, op->init_guess ? PARARNN_INIT_ZERO : op->init_mode, pb->T);
}

// the agreement bar of the K*(T) table (max abs against the unroll)
constexpr float kKStarTau = 1e-4f;

// Iterations per launch of a solve's fused passes (1: one launch per iteration).  Fixed budget: all
// K iterations, PARARNN_MAX_FUSE at a time.  Tolerance mode: the first pass runs speculatively (a
// re-run corrects it when the stop came earlier; single launches follow when it came later) for the
// iteration count tolerance mode reached on the K*(T) campaign's inputs at the nearest of its
// tolerances at or above tol (stop_iters: K*(T) + 1 or K*(T) + 2 on every cell, first iterate and length
// of the grid), or K*(T) when tol is looser than the table's 1e-4 agreement bar.  Speculating short costs
// a single launch per missing iteration, speculating long a re-run of the pass, so the bracket's looser
// end is taken.  opts->fuse_iters overrides the length; Picard sweeps and the cells without a fused
// kernel run one launch per iteration.  NULL opts: the longest pass any options can ask for (the
// workspace size that fits every solve of the problem).
int fuse_len(const pararnn_problem* pb, const pararnn_newton_opts* op) {
  if (!pick_newton(pb).fused) return 1;
  if (!op) return PARARNN_MAX_FUSE;
  if (op->picard_iters > 0 || op->fuse_iters == 1) return 1;
  const int K = budget(pb, op);
  int m = PARARNN_MAX_FUSE;
  if (op->fuse_iters > 1) m = op->fuse_iters;
  else if (op->tol > 0.0f) {
    const int init = op->init_guess ? PARARNN_INIT_ZERO : op->init_mode;
    m = op->tol <= kKStarTau ? stop_iters(pb->cell, init, pb->T, op->tol) : auto_iters(pb->cell, init, pb->T);
  }
  m = std::min(m, std::min(K, PARARNN_MAX_FUSE));
  return m < 1 ? 1 : m;
}

// the arguments of a Newton entry point other than its workspace
pararnn_status newton_check_args(const pararnn_problem* pb, const pararnn_newton_opts* op, const float* s_out,
                                 bool need_out) {
  pararnn_status rc = check_problem(pb);
  if (rc) return rc;
  if (!op || op->max_iters < 0 || op->max_iters > PARARNN_MAX_ITERS) return PARARNN_ERR_INVALID_ARG;
  if (op->init_mode != PARARNN_INIT_ZERO && op->init_mode != PARARNN_INIT_WARM) return PARARNN_ERR_INVALID_ARG;
  if (op->picard_iters < 0 || op->picard_iters > PARARNN_MAX_ITERS) return PARARNN_ERR_INVALID_ARG;
  if (op->fuse_iters < 0 || op->fuse_iters > PARARNN_MAX_FUSE) return PARARNN_ERR_INVALID_ARG;
  if (op->max_iters == 0 && (pb->cell == CELL_SLSTM || pb->cell == CELL_HEAD_GRU))
    return PARARNN_ERR_INVALID_ARG;   // no measured budget
  if (problem_N(pb) == 0) return PARARNN_OK;
  if (need_out && (!s_out || !aligned(s_out, 8))) return PARARNN_ERR_INVALID_ARG;
  if (op->init_guess && !aligned(op->init_guess, 8)) return PARARNN_ERR_INVALID_ARG;
  return PARARNN_OK;
}

pararnn_status newton_check(const pararnn_problem* pb, const pararnn_newton_opts* op, const float* s_out,
                            bool need_out, void* ws, size_t ws_bytes) {
  pararnn_status rc = newton_check_args(pb, op, s_out, need_out);
  if (rc || problem_N(pb) == 0) return rc;
  if (!ws || !aligned(ws, 256) || ws_bytes < pick_newton(pb).ws(pb, fuse_len(pb, op))) return PARARNN_ERR_WORKSPACE;
  return PARARNN_OK;
}

bool overlap(const void* p, const void* q, size_t n) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + n && b < a + n;
}
}  // namespace

size_t pararnn_newton_workspace_bytes(const pararnn_problem* pb, const pararnn_newton_opts* op) {
  if (check_problem(pb) != PARARNN_OK) return 0;
  if (problem_N(pb) == 0) return kHeader;
  return pick_newton(pb).ws(pb, fuse_len(pb, op));
}

pararnn_status pararnn_newton_prepare(const pararnn_problem* pb, const pararnn_newton_opts* op, void* ws,
                                      size_t ws_bytes, void* stream) {
  pararnn_status rc = newton_check(pb, op, nullptr, false, ws, ws_bytes);
  if (rc || problem_N(pb) == 0) return rc;
  return pick_newton(pb).prepare(pb, ws, fuse_len(pb, op), static_cast<hipStream_t>(stream));
}

pararnn_status pararnn_newton_iterate(const pararnn_problem* pb, const pararnn_newton_opts* op, int k, float* s_out,
                                      void* ws, size_t ws_bytes, void* stream) {
  pararnn_status rc = newton_check(pb, op, s_out, true, ws, ws_bytes);
  if (rc || problem_N(pb) == 0) return rc;
  if (k < 0 || k >= budget(pb, op)) return PARARNN_ERR_INVALID_ARG;
  return pick_newton(pb).iterate(pb, op, k, s_out, ws, static_cast<hipStream_t>(stream));
}

pararnn_status pararnn_newton_report(const pararnn_problem* pb, const pararnn_newton_opts* op, const float* s_out,
                                     void* ws, size_t ws_bytes, void* stream, pararnn_report* report) {
  pararnn_status rc = newton_check(pb, op, s_out, op && op->final_residual, ws, ws_bytes);
  if (rc) return rc;
  if (report) std::memset(report, 0, sizeof(*report));
  if (problem_N(pb) == 0) {
    if (report) report->converged = op->tol > 0.0f ? 1 : 0;
    return PARARNN_OK;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (op->final_residual) {
    rc = pick_newton(pb).final_residual(pb, s_out, ws, st);
    if (rc) return rc;
  }
  if (!report) return PARARNN_OK;
  uint32_t res[PARARNN_MAX_ITERS + 1];
  if (hipMemcpyAsync(res, static_cast<char*>(ws) + kResOffset, sizeof(res), hipMemcpyDeviceToHost, st) != hipSuccess)
    return PARARNN_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return PARARNN_ERR_HIP;
  const int K = budget(pb, op);
  int iters = K, conv = 0;
  pararnn_status out = PARARNN_OK;
  for (int k = 0; k < K; ++k) {
    float r;
    std::memcpy(&r, &res[k], sizeof r);
    report->residual[k] = r;
    if (op->tol > 0.0f) {
      if (!(r >= 0.0f) || r == INFINITY) { iters = k + 1; out = PARARNN_ERR_DIVERGED; break; }
      if (r < op->tol) { iters = k + 1; conv = 1; break; }
    }
  }
  // tolerance mode, the budget spent without convergence: a last residual above the one of the iterate
  // Newton started from (after the Picard sweeps) is divergence too
  const int k0 = op->picard_iters;
  if (op->tol > 0.0f && out == PARARNN_OK && !conv && iters - 1 > k0 && report->residual[iters - 1] > report->residual[k0])
    out = PARARNN_ERR_DIVERGED;
  for (int k = iters; k < K; ++k) report->residual[k] = 0.0f;
  report->iters = iters;
  report->converged = conv;
  report->n_residual = iters;
  if (op->final_residual) {
    float r;
    std::memcpy(&r, &res[PARARNN_MAX_ITERS], sizeof r);
    report->residual[iters] = r;
    report->n_residual = iters + 1;
  }
  return out;
}

pararnn_status pararnn_newton_solve(const pararnn_problem* pb, const pararnn_newton_opts* op, float* s_out, void* ws,
                                    size_t ws_bytes, void* stream, pararnn_report* report) {
  pararnn_status rc = newton_check(pb, op, s_out, true, ws, ws_bytes);
  if (rc) return rc;
  if (problem_N(pb) == 0) return pararnn_newton_report(pb, op, s_out, ws, ws_bytes, stream, report);
  const NewtonEntry ne = pick_newton(pb);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int m = fuse_len(pb, op);
  rc = ne.prepare(pb, ws, m, st);
  const int K = budget(pb, op);
  const size_t traj = static_cast<size_t>(state_size(pb->cell)) * problem_N(pb) * sizeof(float);
  if (m <= 1 || (op->tol > 0.0f && op->init_guess && overlap(op->init_guess, s_out, traj))) {
    // one launch per iteration (a speculative pass could not be re-run: s_out overwrites its start)
    const int tail = (op->tol > 0.0f && !ne.fused && ne.iterate_tail) ? op->picard_iters + PR_TAIL_FROM : K;
    for (int k = 0; k < K && rc == PARARNN_OK; ++k)
      rc = k >= tail ? ne.iterate_tail(pb, op, k, s_out, ws, st) : ne.iterate(pb, op, k, s_out, ws, st);
  } else if (op->tol > 0.0f) {
    // speculative pass of m iterations, its re-run if the stop rule met an earlier one, then single
    // launches that exit at once once the stop rule is met.  The re-run and the launches after the first
    // single one mostly find nothing to do and take tickets in a loop on a grid of what is resident (a few
    // us then, against ~15 us for one workgroup per tile; ~3% and ~11% slower when they do run); the first
    // single launch, the one a speculation one short needs, keeps one workgroup per tile
    if (rc == PARARNN_OK) rc = ne.fused(pb, op, 0, m, false, s_out, ws, st);
    if (rc == PARARNN_OK) rc = ne.fused(pb, op, 0, m, true, s_out, ws, st);
    for (int k = m; k < K && rc == PARARNN_OK; ++k)
      rc = k == m ? ne.iterate(pb, op, k, s_out, ws, st) : ne.iterate_tail(pb, op, k, s_out, ws, st);
  } else {
    for (int k = 0; k < K && rc == PARARNN_OK; k += m) {
      const int n = std::min(m, K - k);
      rc = n == 1 ? ne.iterate(pb, op, k, s_out, ws, st) : ne.fused(pb, op, k, n, false, s_out, ws, st);
    }
  }
  if (rc) return rc;
  if (!report && !op->final_residual) return PARARNN_OK;
  return pararnn_newton_report(pb, op, s_out, ws, ws_bytes, stream, report);
}

pararnn_status pararnn_newton_solve_noalloc(const pararnn_problem* pb, const pararnn_newton_opts* op, float* s_out,
                                            void* stream, pararnn_report* report) {
  pararnn_status rc = newton_check_args(pb, op, s_out, true);
  if (rc) return rc;
  if (problem_N(pb) == 0) return pararnn_newton_report(pb, op, s_out, nullptr, 0, stream, report);
  // the library's launch length, shortened until its look-back words fit the scratch (the result is the
  // same bit for bit for every launch length); an explicit fuse_iters is taken as given
  pararnn_newton_opts o = *op;
  const NewtonEntry ne = pick_newton(pb);
  if (o.fuse_iters == 0) {
    int m = fuse_len(pb, &o);
    while (m > 1 && ne.ws(pb, m) > PARARNN_NOALLOC_SCRATCH_BYTES) --m;
    o.fuse_iters = m;
  }
  if (ne.ws(pb, fuse_len(pb, &o)) > PARARNN_NOALLOC_SCRATCH_BYTES) return PARARNN_ERR_WORKSPACE;
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc) return rc;
  return pararnn_newton_solve(pb, &o, s_out, ws, PARARNN_NOALLOC_SCRATCH_BYTES, stream, report);
}

int pararnn_newton_budget(int cell, int init_mode, int64_t T, int max_iters) {
  if (cell < CELL_LINEAR || cell > CELL_HEAD_GRU || T < 0 || max_iters < 0 || max_iters > PARARNN_MAX_ITERS)
    return PARARNN_ERR_INVALID_ARG;
  if (max_iters == 0 && (cell == CELL_SLSTM || cell == CELL_HEAD_GRU))
    return PARARNN_ERR_INVALID_ARG;   // no measured budget
  if (init_mode != PARARNN_INIT_ZERO && init_mode != PARARNN_INIT_WARM) return PARARNN_ERR_INVALID_ARG;
  return max_iters > 0 ? max_iters : auto_iters(cell, init_mode, T);
}

size_t pararnn_scan_workspace_bytes(int S, int64_t B, int64_t T, int64_t D) {
  if ((S != 1 && S != 2) || !sizes_fit(B, T, D)) return 0;
  if (B * T * D == 0) return kHeader;
  return pick_scan(S, PARARNN_F32, 0, false).ws(B, T, D);
}

pararnn_status pararnn_linear_scan(int S, int64_t B, int64_t T, int64_t D, int dtype, const void* a, const void* b,
                                   const float* s0, const int32_t* cu_seqlens, int64_t n_seqs, float* s_out,
                                   int reverse, void* ws, size_t ws_bytes, void* stream) {
  if ((S != 1 && S != 2) || !sizes_fit(B, T, D)) return PARARNN_ERR_INVALID_ARG;
  if (dtype != PARARNN_F32 && dtype != PARARNN_BF16) return PARARNN_ERR_INVALID_ARG;
  if (B * T * D == 0) return PARARNN_OK;
  if (!a || !b || !s_out) return PARARNN_ERR_INVALID_ARG;
  if (!aligned(a, 4) || !aligned(b, 4) || !aligned(s_out, 4) || (s0 && !aligned(s0, 4))) return PARARNN_ERR_INVALID_ARG;
  if (cu_seqlens && (!aligned(cu_seqlens, 4) || n_seqs < 0 || n_seqs > kMaxSeqs)) return PARARNN_ERR_INVALID_ARG;
  const ScanEntry se = pick_scan(S, dtype, reverse ? 1 : 0, cu_seqlens != nullptr);
  if (!ws || !aligned(ws, 256) || ws_bytes < se.ws(B, T, D)) return PARARNN_ERR_WORKSPACE;
  return se.run(B, T, D, a, b, s0, cu_seqlens, n_seqs, s_out, ws, static_cast<hipStream_t>(stream));
}

size_t pararnn_vjp_workspace_bytes(const pararnn_problem* pb) {
  if (check_problem(pb) != PARARNN_OK) return 0;
  if (problem_N(pb) == 0) return kHeader;
  return pick_vjp(pb).ws(pb);
}

pararnn_status pararnn_scan_vjp(const pararnn_problem* pb, const float* s, const float* g, float* d_pre, float* d_w,
                                float* d_bias, float* d_s0, float* lambda_out, void* ws, size_t ws_bytes,
                                void* stream) {
  pararnn_status rc = check_problem(pb);
  if (rc) return rc;
  if (problem_N(pb) == 0) return PARARNN_OK;
  if (!s || !g || !d_pre || !aligned(s, 8) || !aligned(g, 8) || !aligned(d_pre, 8)) return PARARNN_ERR_INVALID_ARG;
  if ((lambda_out && !aligned(lambda_out, 8)) || (d_s0 && !aligned(d_s0, 8))) return PARARNN_ERR_INVALID_ARG;
  const VjpEntry ve = pick_vjp(pb);
  if (!ws || !aligned(ws, 256) || ws_bytes < ve.ws(pb)) return PARARNN_ERR_WORKSPACE;
  return ve.run(pb, s, g, d_pre, d_w, d_bias, d_s0, lambda_out, ws, static_cast<hipStream_t>(stream));
}

#if PR_LB_STRESS
// (libraries built with -DPR_LB_STRESS=1 only; declared in pararnn_debug.h)
int pararnn_debug_lookback_depth(int reset) {
  uint32_t d = 0;
  if (hipDeviceSynchronize() != hipSuccess) return PARARNN_ERR_HIP;
  if (hipMemcpyFromSymbol(&d, HIP_SYMBOL(pr::g_lb_max_depth), sizeof d) != hipSuccess) return PARARNN_ERR_HIP;
  if (reset) {
    const uint32_t z = 0;
    if (hipMemcpyToSymbol(HIP_SYMBOL(pr::g_lb_max_depth), &z, sizeof z) != hipSuccess) return PARARNN_ERR_HIP;
  }
  return static_cast<int>(d);
}
#endif

}  // extern "C"
