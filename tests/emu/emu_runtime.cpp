// Host runtime behind hip_cpu.h: fibers for GPU threads, workgroup barriers, 64-lane wave
// operations (ballot, readlane, shuffles, the DPP row shifts and broadcasts the scans use,
// the gfx950 lane swaps, v_mfma_f32_16x16x128_f8f6f4 on OCP E4M3FN operands), poisoned LDS at
// every workgroup start, and stream capture into replayable graphs.  Test infrastructure only.
#include <sanitizer/common_interface_defs.h>
#include <sys/mman.h>
#if defined(EMU_TSAN)
#include <sanitizer/tsan_interface.h>
#endif

#include <random>

#include "hip_cpu.h"

// x86-64 context switch: saves callee-saved registers on the current stack, stores its stack
// pointer to *save and continues on `next`.
extern "C" void emu_switch(void **save, void *next);
asm(R"(
.text
.globl emu_switch
.type emu_switch,@function
emu_switch:
  pushq %rbp
  pushq %rbx
  pushq %r12
  pushq %r13
  pushq %r14
  pushq %r15
  movq %rsp, (%rdi)
  movq %rsi, %rsp
  popq %r15
  popq %r14
  popq %r13
  popq %r12
  popq %rbx
  popq %rbp
  ret
.size emu_switch,.-emu_switch
)");

namespace emu {

enum { RUN = 0, AT_BARRIER = 1, AT_WAVE = 2, DONE = 3 };

struct Fiber {
  void *sp = nullptr;
  char *stack = nullptr;
  Ctx ctx;
  int state = DONE;
  void *fake = nullptr;
};

constexpr size_t STACK = 512 * 1024;
constexpr int MAXT = 1024;
constexpr int SLOT = 256;

struct Wave {
  int arrived = 0;
  const void *op = nullptr;
  bool divergent = false;
  unsigned char in[64][SLOT];
  unsigned char out[64][SLOT];
};

static Fiber g_f[MAXT];
static Wave g_w[MAXT / 64];
static int g_n = 0, g_live = 0, g_bar = 0;
static Fiber *g_cur = nullptr;
static void *g_sched_sp = nullptr;
static const void *g_sched_bottom = nullptr;
static size_t g_sched_size = 0;
static std::function<void()> *g_body = nullptr;
static bool g_capturing = false;
static std::vector<std::function<void()>> g_capture;
static long long g_launches = 0;

// ECHO_EMU_ORDER=<nonzero seed>: workgroups of a launch run in a seeded random order, and the
// waves of a workgroup are taken in a fresh random order at every scheduling pass (lanes of a
// wave stay in ascending order, as their lockstep execution is not modelled), so a result
// that depends on the order of workgroups or waves shows up as a difference between seeds.
static const unsigned long g_order_seed = [] {
  const char *e = getenv("ECHO_EMU_ORDER");
  return e ? strtoul(e, nullptr, 10) : 0ul;
}();
static std::mt19937 g_rng(static_cast<unsigned>(g_order_seed));

Ctx *ctx() { return &g_cur->ctx; }

// ---- sanitizer views of the fibers
// AddressSanitizer is told about every stack switch.  ThreadSanitizer sees one fiber per wave
// (its lanes run in lockstep on the GPU, so they are one thread of execution): switches carry
// no ordering of their own, workgroup barriers are release/acquire edges between the waves,
// and the start and end of a workgroup are ordered with the host thread, so the check finds
// memory shared by waves of one workgroup without a barrier in between.
#if defined(EMU_TSAN)
static void *g_tsan_host = nullptr;
static void *g_tsan_wave[MAXT / 64];
static char g_tsan_barrier;
static void tsan_enter(int wave, bool sync) {
  __tsan_switch_to_fiber(g_tsan_wave[wave], sync ? 0 : __tsan_switch_to_fiber_no_sync);
}
static void tsan_leave(bool sync) { __tsan_switch_to_fiber(g_tsan_host, sync ? 0 : __tsan_switch_to_fiber_no_sync); }
#else
static void tsan_enter(int, bool) {}
static void tsan_leave(bool) {}
#endif
#if defined(EMU_ASAN)
static void asan_start(void **fake, const void *bottom, size_t size) { __sanitizer_start_switch_fiber(fake, bottom, size); }
static void asan_finish(void *fake, const void **bottom, size_t *size) { __sanitizer_finish_switch_fiber(fake, bottom, size); }
#else
static void asan_start(void **, const void *, size_t) {}
static void asan_finish(void *, const void **, size_t *) {}
#endif

[[noreturn]] static void die(const char *msg) {
  fprintf(stderr, "EMU ERROR: %s (workgroup %u,%u thread %u)\n", msg, g_cur ? g_cur->ctx.bid.x : 0,
          g_cur ? g_cur->ctx.bid.y : 0, g_cur ? g_cur->ctx.tid.x : 0);
  fflush(stderr);
  abort();
}

// LDS poisoning: every __shared__ object registers itself when a thread first passes its
// declaration; its bytes are overwritten with POISON then and at the start of every later
// workgroup, so a read of LDS that the workgroup did not write yields garbage, as on the GPU.
constexpr unsigned char POISON = 0xBE;
struct LdsRegion { void *p; size_t n; };
static std::vector<LdsRegion> g_lds;

void lds_register(void *p, size_t n) {
  for (const auto &r : g_lds)
    if (r.p == p) return;
  g_lds.push_back({p, n});
  memset(p, POISON, n);
}

const void *device_symbol(const void *p, size_t n) {
  static std::vector<const void *> seen;
  for (const void *q : seen)
    if (q == p) return p;
  seen.push_back(p);
  memset(const_cast<void *>(p), POISON, n);
  return p;
}

static void poison_lds() {
  for (const auto &r : g_lds) memset(r.p, POISON, r.n);
}

static void to_sched() {
  asan_start(&g_cur->fake, g_sched_bottom, g_sched_size);
  tsan_leave(false);
  emu_switch(&g_cur->sp, g_sched_sp);
  asan_finish(g_cur->fake, nullptr, nullptr);
}

static void release_barrier_if_complete() {
  if (g_live > 0 && g_bar == g_live) {
    for (int i = 0; i < g_n; ++i)
      if (g_f[i].state == AT_BARRIER) g_f[i].state = RUN;
    g_bar = 0;
  }
}

static void fiber_entry() {
  asan_finish(nullptr, &g_sched_bottom, &g_sched_size);
  (*g_body)();
  g_cur->state = DONE;
  --g_live;
  // a wave whose other lanes wait in a wave op can never complete now
  Wave &w = g_w[g_cur->ctx.wave];
  if (w.arrived > 0) die("a lane ended while the rest of its wave waits in a wave op");
  release_barrier_if_complete();
  asan_start(nullptr, g_sched_bottom, g_sched_size);
  tsan_leave(true);                       // the host thread continues after the whole workgroup
  void *dead;
  emu_switch(&dead, g_sched_sp);
  abort();
}

void barrier() {
  if (g_w[g_cur->ctx.wave].arrived > 0) die("barrier while lanes of this wave wait in a wave op");
#if defined(EMU_TSAN)
  __tsan_release(&g_tsan_barrier);
#endif
  g_cur->state = AT_BARRIER;
  ++g_bar;
  release_barrier_if_complete();
  if (g_cur->state == AT_BARRIER) to_sched();
#if defined(EMU_TSAN)
  __tsan_acquire(&g_tsan_barrier);
#endif
}

static int live_lanes(int wave) {
  int c = 0;
  for (int l = 0; l < 64; ++l) {
    const int i = wave * 64 + l;
    if (i < g_n && g_f[i].state != DONE) ++c;
  }
  return c;
}

void wave_op(const void *in, size_t ib, void *out, size_t ob,
             void (*fn)(const unsigned char *, unsigned char *, size_t, size_t, const void *),
             const void *arg) {
  if (ib > SLOT || ob > SLOT) die("wave op payload too large");
  const int wv = g_cur->ctx.wave, l = g_cur->ctx.lane;
  Wave &w = g_w[wv];
  if (w.arrived == 0) { w.op = reinterpret_cast<const void *>(fn); w.divergent = false; }
  else if (w.op != reinterpret_cast<const void *>(fn)) w.divergent = true;
  memcpy(w.in[l], in, ib);
  ++w.arrived;
  if (w.arrived == 64) {
    if (w.divergent) die("lanes of one wave met different wave ops");
    fn(&w.in[0][0], &w.out[0][0], ib, ob, arg);
    w.arrived = 0;
    for (int j = 0; j < 64; ++j)
      if (g_f[wv * 64 + j].state == AT_WAVE) g_f[wv * 64 + j].state = RUN;
  } else {
    if (live_lanes(wv) < 64) die("wave op with inactive lanes (exec mask not full)");
    g_cur->state = AT_WAVE;
    to_sched();
  }
  memcpy(out, w.out[l], ob);
}

static void run_block(dim3 grid, dim3 block, dim3 bid) {
  const int n = static_cast<int>(block.x * block.y * block.z);
  if (n > MAXT || n < 1) die("block size must be 1..1024");
  g_n = n;
  g_live = n;
  g_bar = 0;
  poison_lds();
  for (int i = 0; i < (n + 63) / 64; ++i) g_w[i].arrived = 0;
  for (int i = 0; i < n; ++i) {
    Fiber &f = g_f[i];
    if (!f.stack) {
      f.stack = static_cast<char *>(mmap(nullptr, STACK, PROT_READ | PROT_WRITE, MAP_PRIVATE | MAP_ANONYMOUS | MAP_NORESERVE, -1, 0));
      if (f.stack == MAP_FAILED) die("mmap");
    }
    uintptr_t top = (reinterpret_cast<uintptr_t>(f.stack) + STACK) & ~uintptr_t(15);
    void **sp = reinterpret_cast<void **>(top);
    *--sp = nullptr;                                        // return address of fiber_entry
    *--sp = reinterpret_cast<void *>(&fiber_entry);         // popped by emu_switch's ret
    for (int r = 0; r < 6; ++r) *--sp = nullptr;            // callee-saved registers
    f.sp = sp;
    f.ctx.tid = dim3(i % block.x, (i / block.x) % block.y, i / (block.x * block.y));
    f.ctx.bid = bid;
    f.ctx.bdim = block;
    f.ctx.gdim = grid;
    f.ctx.lane = i % 64;
    f.ctx.wave = i / 64;
    f.state = RUN;
    f.fake = nullptr;
  }
  const int n_waves = (n + 63) / 64;
#if defined(EMU_TSAN)
  g_tsan_host = __tsan_get_current_fiber();
  for (int v = 0; v < n_waves; ++v) g_tsan_wave[v] = __tsan_create_fiber(0);
#endif
  bool started[MAXT];
  for (int i = 0; i < n; ++i) started[i] = false;
  int worder[MAXT / 64];
  for (int v = 0; v < n_waves; ++v) worder[v] = v;
  while (g_live > 0) {
    bool progress = false;
    if (g_order_seed) std::shuffle(worder, worder + n_waves, g_rng);
    for (int ii = 0; ii < n; ++ii) {
      const int i = worder[ii / 64] * 64 + ii % 64;        // waves in (shuffled) order, lanes ascending
      if (i >= n || g_f[i].state != RUN) continue;
      g_cur = &g_f[i];
      void *fake = nullptr;
      asan_start(&fake, g_cur->stack, STACK);
      tsan_enter(g_cur->ctx.wave, !started[i]);   // the workgroup starts after the host's setup
      started[i] = true;
      emu_switch(&g_sched_sp, g_cur->sp);
      asan_finish(fake, nullptr, nullptr);
      progress = true;
    }
    if (!progress && g_live > 0) {
      release_barrier_if_complete();
      bool any = false;
      for (int i = 0; i < n; ++i) any |= g_f[i].state == RUN;
      if (!any) { g_cur = &g_f[0]; die("deadlock: no runnable thread (barrier / wave-op mismatch)"); }
    }
  }
#if defined(EMU_TSAN)
  for (int v = 0; v < n_waves; ++v) __tsan_destroy_fiber(g_tsan_wave[v]);
#endif
  g_cur = nullptr;
}

void launch(dim3 grid, dim3 block, std::function<void()> body) {
  if (g_capturing) {
    g_capture.push_back([grid, block, body]() { launch(grid, block, body); });
    return;
  }
  ++g_launches;
  std::function<void()> b = body;
  g_body = &b;
  std::vector<dim3> blocks;
  for (uint32_t z = 0; z < grid.z; ++z)
    for (uint32_t y = 0; y < grid.y; ++y)
      for (uint32_t x = 0; x < grid.x; ++x) blocks.push_back(dim3(x, y, z));
  if (g_order_seed) std::shuffle(blocks.begin(), blocks.end(), g_rng);
  for (const dim3 &bid : blocks) run_block(grid, block, bid);
  g_body = nullptr;
}

void set_capture(bool on) { g_capturing = on; if (on) g_capture.clear(); }
std::vector<std::function<void()>> take_capture() { auto v = std::move(g_capture); g_capture.clear(); return v; }

// ---------------------------------------------------------------- op kernels
static void op_ballot(const unsigned char *in, unsigned char *out, size_t, size_t, const void *) {
  unsigned long long m = 0;
  for (int l = 0; l < 64; ++l) if (in[l * SLOT]) m |= 1ull << l;
  for (int l = 0; l < 64; ++l) memcpy(out + l * SLOT, &m, 8);
}
struct IdxIn { int v; int idx; };
static void op_readlane(const unsigned char *in, unsigned char *out, size_t, size_t, const void *) {
  IdxIn a;
  memcpy(&a, in, sizeof a);
  const int lane = a.idx;
  for (int l = 0; l < 64; ++l) {
    IdxIn b;
    memcpy(&b, in + l * SLOT, sizeof b);
    if (b.idx != lane) { fprintf(stderr, "EMU ERROR: readlane with a non-uniform lane\n"); abort(); }
  }
  if (lane < 0 || lane > 63) { fprintf(stderr, "EMU ERROR: readlane lane %d\n", lane); abort(); }
  IdxIn src;
  memcpy(&src, in + lane * SLOT, sizeof src);
  for (int l = 0; l < 64; ++l) memcpy(out + l * SLOT, &src.v, 4);
}
static void op_shfl(const unsigned char *in, unsigned char *out, size_t, size_t, const void *arg) {
  const int mode = *static_cast<const int *>(arg);   // 0: xor, 1: direct
  for (int l = 0; l < 64; ++l) {
    IdxIn a;
    memcpy(&a, in + l * SLOT, sizeof a);
    const int src = mode == 0 ? (l ^ a.idx) : a.idx;
    if (src < 0 || src > 63) { fprintf(stderr, "EMU ERROR: shuffle source %d\n", src); abort(); }
    IdxIn b;
    memcpy(&b, in + src * SLOT, sizeof b);
    memcpy(out + l * SLOT, &b.v, 4);
  }
}
struct DppIn { int old, src, ctrl, row_mask, bank_mask, bc; };
static void op_dpp(const unsigned char *in, unsigned char *out, size_t, size_t, const void *) {
  DppIn a0;
  memcpy(&a0, in, sizeof a0);
  for (int l = 0; l < 64; ++l) {
    DppIn a;
    memcpy(&a, in + l * SLOT, sizeof a);
    if (a.ctrl != a0.ctrl || a.row_mask != a0.row_mask || a.bank_mask != a0.bank_mask || a.bc != a0.bc) {
      fprintf(stderr, "EMU ERROR: non-uniform DPP control\n");
      abort();
    }
    const int row = l / 16, rl = l % 16;
    int src = -1;
    if (a.ctrl >= 0x111 && a.ctrl <= 0x11F) { const int s = a.ctrl - 0x110; if (rl >= s) src = l - s; }
    else if (a.ctrl == 0x142) { if (row >= 1) src = 16 * row - 1; }
    else if (a.ctrl == 0x143) { if (row >= 2) src = 31; }
    else { fprintf(stderr, "EMU ERROR: DPP control 0x%x not emulated\n", a.ctrl); abort(); }
    const bool enabled = ((a.row_mask >> row) & 1) && ((a.bank_mask >> (rl / 4)) & 1);
    int v = a.old;
    if (enabled) {
      if (src >= 0) { DppIn s; memcpy(&s, in + src * SLOT, sizeof s); v = s.src; }
      else if (a.bc) v = 0;
    }
    memcpy(out + l * SLOT, &v, 4);
  }
}
// v_permlane32_swap exchanges the upper 32 lanes of its first operand with the lower 32 lanes
// of its second; v_permlane16_swap exchanges the odd 16-lane rows of the first with the even
// rows of the second.  The builtins return {first, second} after the exchange.
struct SwapIn { unsigned a, b; };
// ECHO_EMU_SWAP_FLIP (bits 0 / 1) reverses the 16 / 32-lane exchange (first operand's even rows
// with the second's odd rows; first operand's lower half with the second's upper half), to
// check code that must not depend on the direction.
static const int g_swap_flip = [] {
  const char *e = getenv("ECHO_EMU_SWAP_FLIP");
  return e ? atoi(e) : 0;
}();

static void op_swap(const unsigned char *in, unsigned char *out, size_t, size_t, const void *arg) {
  const int which = *static_cast<const int *>(arg);   // 16 or 32
  const bool flip = (g_swap_flip >> (which == 32 ? 1 : 0)) & 1;
  for (int l = 0; l < 64; ++l) {
    SwapIn s;
    memcpy(&s, in + l * SLOT, sizeof s);
    unsigned na = s.a, nb = s.b;
    SwapIn o;
    if (which == 32) {
      const bool upper = l >= 32;
      if (upper != flip) { memcpy(&o, in + (upper ? l - 32 : l + 32) * SLOT, sizeof o); na = o.b; }
      else { memcpy(&o, in + (upper ? l - 32 : l + 32) * SLOT, sizeof o); nb = o.a; }
    } else {
      const bool odd = (l / 16) & 1;
      if (odd != flip) { memcpy(&o, in + (odd ? l - 16 : l + 16) * SLOT, sizeof o); na = o.b; }
      else { memcpy(&o, in + (odd ? l - 16 : l + 16) * SLOT, sizeof o); nb = o.a; }
    }
    const unsigned r[2] = {na, nb};
    memcpy(out + l * SLOT, r, 8);
  }
}
// OCP E4M3FN: bias 7, no infinities, S.1111.111 is NaN, exponent 0 is subnormal.
static float e4m3fn(unsigned char b) {
  const int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  if (e == 15 && m == 7) return NAN;
  const float v = e == 0 ? std::ldexp(static_cast<float>(m), -9) : std::ldexp(1.0f + m / 8.0f, e - 7);
  return s ? -v : v;
}
// 16x16x128 fp8 MFMA: lane l supplies row l%16 of A and column l%16 of B for K bytes
// [32 (l/16), 32 (l/16) + 32); the result C[4 (l/16) + v][l%16] lands in lane l, element v.
// Products of two fp8 values and their sums over K are exact in double; the hardware's fp32
// accumulation can differ from this in the last bits for general inputs.
struct MfmaIn { v8i_emu a, b; v4f_emu c; };
static void op_mfma(const unsigned char *in, unsigned char *out, size_t, size_t, const void *) {
  static float tab[256];
  static bool init = false;
  if (!init) { for (int i = 0; i < 256; ++i) tab[i] = e4m3fn(static_cast<unsigned char>(i)); init = true; }
  unsigned char A[16][128], B[128][16];
  for (int l = 0; l < 64; ++l) {
    MfmaIn x;
    memcpy(&x, in + l * SLOT, sizeof x);
    const int j = l % 16, g = l / 16;
    unsigned char ab[32], bb[32];
    memcpy(ab, &x.a, 32);
    memcpy(bb, &x.b, 32);
    for (int q = 0; q < 32; ++q) { A[j][32 * g + q] = ab[q]; B[32 * g + q][j] = bb[q]; }
  }
  for (int l = 0; l < 64; ++l) {
    MfmaIn x;
    memcpy(&x, in + l * SLOT, sizeof x);
    const int j = l % 16, g = l / 16;
    v4f_emu r;
    for (int v = 0; v < 4; ++v) {
      const int i = 4 * g + v;
      double acc = 0;
      for (int k = 0; k < 128; ++k) acc += static_cast<double>(tab[A[i][k]]) * tab[B[k][j]];
      r[v] = static_cast<float>(acc + x.c[v]);
    }
    memcpy(out + l * SLOT, &r, 16);
  }
}

}  // namespace emu

using namespace emu;

unsigned long long __ballot(bool pred) {
  unsigned char p = pred ? 1 : 0;
  unsigned long long r;
  wave_op(&p, 1, &r, 8, op_ballot, nullptr);
  return r;
}
// __builtin_amdgcn_wave_barrier: on the GPU only a compiler ordering point, since a wave's LDS
// operations execute in order; here the lanes of the wave meet, so an LDS word one lane wrote
// before it is seen by the others after it, as in lockstep execution.
static void op_none(const unsigned char *, unsigned char *, size_t, size_t, const void *) {}
void emu_amdgcn_wave_barrier() {
  unsigned char p = 0, r;
  wave_op(&p, 1, &r, 1, op_none, nullptr);
}
int emu_readlane_i(int v, int lane) {
  IdxIn a{v, lane};
  int r;
  wave_op(&a, sizeof a, &r, 4, op_readlane, nullptr);
  return r;
}
static int shfl_i(int v, int idx, int mode) {
  static const int modes[2] = {0, 1};
  IdxIn a{v, idx};
  int r;
  wave_op(&a, sizeof a, &r, 4, op_shfl, &modes[mode]);
  return r;
}
float __shfl_xor(float v, int mask, int) { return __int_as_float(shfl_i(__float_as_int(v), mask, 0)); }
int __shfl_xor(int v, int mask, int) { return shfl_i(v, mask, 0); }
unsigned __shfl_xor(unsigned v, int mask, int) { return static_cast<unsigned>(shfl_i(static_cast<int>(v), mask, 0)); }
float __shfl(float v, int lane, int) { return __int_as_float(shfl_i(__float_as_int(v), lane, 1)); }
int __shfl(int v, int lane, int) { return shfl_i(v, lane, 1); }
unsigned __shfl(unsigned v, int lane, int) { return static_cast<unsigned>(shfl_i(static_cast<int>(v), lane, 1)); }
int emu_amdgcn_update_dpp(int old, int src, int ctrl, int row_mask, int bank_mask, bool bc) {
  DppIn a{old, src, ctrl, row_mask, bank_mask, bc ? 1 : 0};
  int r;
  wave_op(&a, sizeof a, &r, 4, op_dpp, nullptr);
  return r;
}
v2u_emu emu_amdgcn_permlane16_swap(unsigned a, unsigned b, bool, bool) {
  static const int w = 16;
  SwapIn s{a, b};
  unsigned r[2];
  wave_op(&s, sizeof s, r, 8, op_swap, &w);
  return v2u_emu{r[0], r[1]};
}
v2u_emu emu_amdgcn_permlane32_swap(unsigned a, unsigned b, bool, bool) {
  static const int w = 32;
  SwapIn s{a, b};
  unsigned r[2];
  wave_op(&s, sizeof s, r, 8, op_swap, &w);
  return v2u_emu{r[0], r[1]};
}
v4f_emu emu_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(v8i_emu a, v8i_emu b, v4f_emu c, int, int, int, int, int, int) {
  MfmaIn x{a, b, c};
  v4f_emu r;
  wave_op(&x, sizeof x, &r, 16, op_mfma, nullptr);
  return r;
}

// ---------------------------------------------------------------- host runtime
struct emu_graph { std::vector<std::function<void()>> nodes; };
hipError_t hipGetLastError() { return hipSuccess; }
const char *hipGetErrorString(hipError_t e) { return e ? "emulated error" : "no error"; }
hipError_t hipMemcpy(void *d, const void *s, size_t n, int) { memmove(d, s, n); return hipSuccess; }
hipError_t hipMemcpyAsync(void *d, const void *s, size_t n, int, hipStream_t) {
  if (g_capturing) { g_capture.push_back([d, s, n]() { memmove(d, s, n); }); return hipSuccess; }
  memmove(d, s, n);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipStreamBeginCapture(hipStream_t, int) { set_capture(true); return hipSuccess; }
hipError_t hipStreamEndCapture(hipStream_t, hipGraph_t *g) {
  set_capture(false);
  *g = new emu_graph{take_capture()};
  return hipSuccess;
}
hipError_t hipGraphInstantiate(hipGraphExec_t *e, hipGraph_t g, void *, void *, size_t) {
  *e = new emu_graph{g->nodes};
  return hipSuccess;
}
hipError_t hipGraphLaunch(hipGraphExec_t e, hipStream_t) {
  for (auto &n : e->nodes) n();
  return hipSuccess;
}
hipError_t hipGraphDestroy(hipGraph_t g) { delete g; return hipSuccess; }
hipError_t hipGraphExecDestroy(hipGraphExec_t e) { delete e; return hipSuccess; }
hipError_t hipHostMalloc(void **p, size_t n, unsigned) { *p = malloc(n); return *p ? hipSuccess : hipErrorInvalidValue; }
hipError_t hipHostGetDevicePointer(void **d, void *h, unsigned) { *d = h; return hipSuccess; }
hipError_t hipHostFree(void *p) { free(p); return hipSuccess; }
hipError_t hipGetDevice(int *d) { *d = 0; return hipSuccess; }
hipError_t hipGetSymbolAddress(void **p, const void *sym) { *p = const_cast<void *>(sym); return hipSuccess; }

extern "C" long long emu_launch_count() { return g_launches; }
