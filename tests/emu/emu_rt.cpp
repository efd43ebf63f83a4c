// Runtime of the CPU emulation of the HIP kernels: a pool of worker threads
// runs the blocks of a grid; inside a block every work-item is a fiber, and
// the scheduler switches fibers only at barriers and wavefront rendezvous
// points.  TEST INFRASTRUCTURE ONLY (see include/hip/hip_runtime.h).
#include <hip/hip_runtime.h>

#include <sys/mman.h>
#include <unistd.h>

#include <atomic>
#include <chrono>
#include <condition_variable>
#include <deque>
#include <mutex>
#include <pthread.h>
#include <string>
#include <thread>
#include <vector>

#if defined(__has_feature)
#if __has_feature(address_sanitizer)
#define EMU_ASAN 1
#include <sanitizer/asan_interface.h>
#include <sanitizer/common_interface_defs.h>
#endif
#endif

extern "C" void emu_switch(void** save_sp, void* load_sp);
extern "C" void emu_fiber_tramp();
extern "C" void emu_fiber_main();

namespace emu {

namespace {

constexpr size_t STACK = 256 * 1024;
constexpr int MAXT = 1024;

enum { RUN = 0, WAIT_BAR = 1, WAIT_WAVE = 2, DEAD = 3 };

struct PendingWrite {
  char* dst;
  unsigned char data[16];
  int n;
};

struct WaveState {
  int alive = 0, arrived = 0, kind = 0;
  CollFn fn = nullptr;
  void* ctx = nullptr;
  std::deque<std::vector<PendingWrite>> q;  // in-flight LDS loads, one group per instruction
};

}  // namespace

struct Fiber {
  void* sp = nullptr;
  dim3 tid;
  int lin = 0, lane = 0, wave = 0, state = DEAD;
  alignas(64) unsigned char in[128];
  alignas(64) unsigned char out[128];
};

namespace {

struct Worker {
  std::vector<Fiber> fibers;
  std::vector<unsigned char*> stacks;
  void* sched_sp = nullptr;
  Fiber* current = nullptr;
  dim3 bid, bdim, gdim;
  int nthreads = 0, nwaves = 0, alive = 0, at_barrier = 0, coll_wave = 0;
  WaveState waves[MAXT / 64];
  std::vector<unsigned char> dyn;
  BlockThunk thunk = nullptr;
  void* args = nullptr;
  Worker() : fibers(MAXT) {}
};

thread_local Worker* W = nullptr;
int g_range_mode = 0;      // 0: scalar offset counted by the range check; 1: not counted
int g_reverse_order = 0;   // schedule lanes and waves in reverse order
int g_land_early = 0;      // buffer-to-LDS writes land at issue instead of at the covering wait
std::atomic<long> g_collectives{0};

[[noreturn]] void fatal(const std::string& m) {
  std::fprintf(stderr, "emu: %s\n", m.c_str());
  std::fflush(stderr);
  std::abort();
}

unsigned char* new_stack() {
  size_t pg = (size_t)sysconf(_SC_PAGESIZE);
  void* p = mmap(nullptr, STACK + pg, PROT_READ | PROT_WRITE, MAP_PRIVATE | MAP_ANONYMOUS, -1, 0);
  if (p == MAP_FAILED) fatal("stack mmap failed");
  mprotect(p, pg, PROT_NONE);  // guard page below the stack
  return (unsigned char*)p + pg;
}

// Stack switches, announced to AddressSanitizer in sanitized builds.
void switch_to_fiber(Fiber& f);
void switch_to_sched(Fiber* f);

void to_sched() { switch_to_sched(W->current); }

void complete_wave(int wave) {
  WaveState& w = W->waves[wave];
  W->coll_wave = wave;
  w.fn(w.ctx);
  ++g_collectives;
  w.arrived = 0;
  for (int l = 0; l < 64; ++l) {
    int i = wave * 64 + l;
    if (i < W->nthreads && W->fibers[i].state == WAIT_WAVE) W->fibers[i].state = RUN;
  }
}

void release_barrier() {
  W->at_barrier = 0;
  for (int i = 0; i < W->nthreads; ++i)
    if (W->fibers[i].state == WAIT_BAR) W->fibers[i].state = RUN;
}

void describe_and_die(const char* what) {
  std::string m = std::string(what) + " in block (" + std::to_string(W->bid.x) + "," +
                  std::to_string(W->bid.y) + "," + std::to_string(W->bid.z) + "); states:";
  for (int wv = 0; wv < W->nwaves; ++wv) {
    int c[4] = {0, 0, 0, 0};
    for (int l = 0; l < 64 && wv * 64 + l < W->nthreads; ++l) c[W->fibers[wv * 64 + l].state]++;
    m += " w" + std::to_string(wv) + "[run " + std::to_string(c[0]) + " bar " + std::to_string(c[1]) +
         " wave " + std::to_string(c[2]) + "(kind " + std::to_string(W->waves[wv].kind) + ") dead " +
         std::to_string(c[3]) + "]";
  }
  fatal(m);
}

void run_block() {
  const int n = W->nthreads;
  while ((int)W->stacks.size() < n) W->stacks.push_back(new_stack());
  W->nwaves = (n + 63) / 64;
  W->alive = n;
  W->at_barrier = 0;
  for (int wv = 0; wv < W->nwaves; ++wv) {
    WaveState& w = W->waves[wv];
    w.alive = std::min(64, n - wv * 64);
    w.arrived = 0;
    w.kind = 0;
    w.q.clear();
  }
  for (int i = 0; i < n; ++i) {
    Fiber& f = W->fibers[i];
    f.lin = i;
    f.lane = i & 63;
    f.wave = i >> 6;
    f.tid = dim3(i % W->bdim.x, (i / W->bdim.x) % W->bdim.y, i / (W->bdim.x * W->bdim.y));
    f.state = RUN;
#ifdef EMU_ASAN
    // A fiber stack is reused block after block, and frames that never
    // returned (a finished fiber's last switch) leave poisoned redzones in
    // its shadow, which later kernels' stack data can land on: start every
    // fiber with a clean shadow, as for any reused stack.
    __asan_unpoison_memory_region(W->stacks[i], STACK);
#endif
    uintptr_t top = ((uintptr_t)(W->stacks[i] + STACK)) & ~(uintptr_t)15;
    void** sp = (void**)top - 8;
    for (int k = 0; k < 6; ++k) sp[k] = nullptr;
    sp[6] = (void*)&emu_fiber_tramp;
    sp[7] = nullptr;
    f.sp = sp;
  }
  while (W->alive > 0) {
    bool ran = false;
    for (int k = 0; k < n; ++k) {
      int i = g_reverse_order ? n - 1 - k : k;
      Fiber& f = W->fibers[i];
      if (f.state != RUN) continue;
      W->current = &f;
      switch_to_fiber(f);
      ran = true;
    }
    if (!ran && W->alive > 0) describe_and_die("deadlock (divergent barrier or wave operation)");
  }
  for (int wv = 0; wv < W->nwaves; ++wv)
    if (!W->waves[wv].q.empty()) {
      // loads never waited for: apply them (the hardware would complete them at wave end)
      for (auto& g : W->waves[wv].q)
        for (auto& pw : g) std::memcpy(pw.dst, pw.data, pw.n);
      W->waves[wv].q.clear();
    }
}

#ifdef EMU_ASAN
thread_local void* t_sched_fake = nullptr;
thread_local const void* t_sched_bottom = nullptr;
thread_local size_t t_sched_size = 0;
#endif

// Protocol of the sanitizer's fiber interface: the side that leaves calls
// start (saving its fake stack, naming the destination stack), the side that
// resumes calls finish (restoring its fake stack, learning the bounds of the
// stack it came from).  Fibers learn the scheduler's stack bounds that way.
void switch_to_fiber(Fiber& f) {
#ifdef EMU_ASAN
  __sanitizer_start_switch_fiber(&t_sched_fake, W->stacks[f.lin], STACK);
  emu_switch(&W->sched_sp, f.sp);
  __sanitizer_finish_switch_fiber(t_sched_fake, nullptr, nullptr);
#else
  emu_switch(&W->sched_sp, f.sp);
#endif
}

void switch_to_sched(Fiber* f) {
#ifdef EMU_ASAN
  void* fake = nullptr;
  __sanitizer_start_switch_fiber(f->state == DEAD ? nullptr : &fake, t_sched_bottom, t_sched_size);
  emu_switch(&f->sp, W->sched_sp);
  __sanitizer_finish_switch_fiber(fake, &t_sched_bottom, &t_sched_size);
#else
  emu_switch(&f->sp, W->sched_sp);
#endif
}

// ------------------------------------------------------------------ worker pool
struct Pool {
  std::vector<std::thread> th;
  std::mutex mu;
  std::condition_variable cv, done_cv;
  long gen = 0;
  int busy = 0;
  std::atomic<long> next{0};
  long nblocks = 0;
  dim3 grid, block;
  size_t shmem = 0;
  BlockThunk thunk = nullptr;
  void* args = nullptr;
  bool stop = false;

  void work() {
    thread_local Worker w;
    W = &w;
    for (;;) {
      long b = next.fetch_add(1);
      if (b >= nblocks) break;
      W->bid = dim3((unsigned)(b % grid.x), (unsigned)((b / grid.x) % grid.y),
                    (unsigned)(b / ((long)grid.x * grid.y)));
      W->bdim = block;
      W->gdim = grid;
      W->nthreads = (int)(block.x * block.y * block.z);
      W->thunk = thunk;
      W->args = args;
      if (W->dyn.size() < shmem) W->dyn.resize(shmem);
      if (shmem) std::memset(W->dyn.data(), 0xFF, shmem);
      run_block();
    }
  }

  void start(int n) {
    for (int i = 0; i < n; ++i)
      th.emplace_back([this] {
        long seen = 0;
        for (;;) {
          {
            std::unique_lock<std::mutex> lk(mu);
            cv.wait(lk, [&] { return stop || gen != seen; });
            if (stop) return;
            seen = gen;
          }
          work();
          {
            std::lock_guard<std::mutex> lk(mu);
            if (--busy == 0) done_cv.notify_all();
          }
        }
      });
  }
};

Pool* pool() {
  static Pool* p = [] {
    Pool* q = new Pool();
    int n = (int)std::thread::hardware_concurrency();
    if (const char* e = std::getenv("EMU_THREADS")) n = std::atoi(e);
    if (n < 1) n = 1;
    if (n > 64) n = 64;
    // Every kernel's LDS arrays are thread_local in this build, and glibc
    // carves static TLS out of each thread's stack: give the workers room
    // (the sanitizer builds' larger frames overflowed the default).
    pthread_attr_t attr;
    if (pthread_getattr_default_np(&attr) == 0) {
      pthread_attr_setstacksize(&attr, (size_t)64 << 20);
      pthread_setattr_default_np(&attr);
      pthread_attr_destroy(&attr);
    }
    q->start(n);
    return q;
  }();
  return p;
}

hipError_t g_last = hipSuccess;

}  // namespace

// ------------------------------------------------------------------ execution context
Fiber* cur() { return W->current; }
const dim3& tid3() { return W->current->tid; }
const dim3& bid3() { return W->bid; }
const dim3& bdim3() { return W->bdim; }
const dim3& gdim3() { return W->gdim; }
void* dyn_shared() { return W->dyn.data(); }
int lane_id() { return W->current->lane; }

const void* lane_in(int lane) {
  int i = W->coll_wave * 64 + lane;
  if (lane < 0 || lane >= 64 || i >= W->nthreads) return nullptr;
  const Fiber& f = W->fibers[i];
  return f.state == DEAD ? nullptr : f.in;
}
void* lane_out(int lane) { return W->fibers[W->coll_wave * 64 + lane].out; }

void* wave_collective(int kind, const void* in, size_t nbytes, CollFn fn, void* ctx) {
  Fiber* f = W->current;
  WaveState& w = W->waves[f->wave];
  if (nbytes > sizeof(f->in)) fatal("collective operand too large");
  std::memcpy(f->in, in, nbytes);
  if (w.arrived == 0) {
    w.kind = kind;
    w.fn = fn;
    w.ctx = ctx;
  } else if (w.kind != kind) {
    fatal("lanes of one wave reached different wave operations (" + std::to_string(w.kind) + " vs " +
          std::to_string(kind) + ")");
  }
  if (++w.arrived == w.alive) {
    complete_wave(f->wave);
  } else {
    f->state = WAIT_WAVE;
    to_sched();
  }
  return f->out;
}

void barrier() {
  Fiber* f = W->current;
  if (++W->at_barrier == W->alive) {
    release_barrier();
  } else {
    f->state = WAIT_BAR;
    to_sched();
  }
}

namespace {
struct WaitCtx {
  int vm;
};
void wait_fn(void* v) {
  WaitCtx* c = (WaitCtx*)v;
  WaveState& w = W->waves[W->coll_wave];
  while ((int)w.q.size() > c->vm) {
    for (auto& pw : w.q.front()) std::memcpy(pw.dst, pw.data, pw.n);
    w.q.pop_front();
  }
}
}  // namespace

void waitcnt(int imm) {
  WaitCtx c{(imm & 0xF) | (((imm >> 14) & 0x3) << 4)};
  wave_collective(1, &c, sizeof(c), wait_fn, &c);
}

void syncthreads() {
  waitcnt(0);
  barrier();
}

// ------------------------------------------------------------------ matrix core
namespace {
struct MfmaIn {
  bf16x8_t a, b;
  f32x16_t c;
};
void mfma_fn(void*) {
  float A[32][16], B[16][32], D[32][32];
  for (int l = 0; l < 64; ++l) {
    const MfmaIn* p = (const MfmaIn*)lane_in(l);
    for (int s = 0; s < 8; ++s) {
      float av = p ? (float)p->a[s] : 0.f, bv = p ? (float)p->b[s] : 0.f;
      A[l & 31][8 * (l >> 5) + s] = av;
      B[8 * (l >> 5) + s][l & 31] = bv;
    }
    for (int e = 0; e < 16; ++e)
      D[8 * (e >> 2) + 4 * (l >> 5) + (e & 3)][l & 31] = p ? p->c[e] : 0.f;
  }
  for (int i = 0; i < 32; ++i)
    for (int k = 0; k < 16; ++k) {
      const float a = A[i][k];
      for (int j = 0; j < 32; ++j) D[i][j] = std::fma(a, B[k][j], D[i][j]);
    }
  for (int l = 0; l < 64; ++l) {
    f32x16_t o;
    for (int e = 0; e < 16; ++e) o[e] = D[8 * (e >> 2) + 4 * (l >> 5) + (e & 3)][l & 31];
    std::memcpy(lane_out(l), &o, sizeof(o));
  }
}
}  // namespace

namespace {
struct MfmaH16In {
  f16x8_t a, b;
  f32x16_t c;
};
void mfma_h16_fn(void*) {
  float A[32][16], B[16][32], D[32][32];
  for (int l = 0; l < 64; ++l) {
    const MfmaH16In* p = (const MfmaH16In*)lane_in(l);
    for (int s = 0; s < 8; ++s) {
      A[l & 31][8 * (l >> 5) + s] = p ? (float)p->a[s] : 0.f;
      B[8 * (l >> 5) + s][l & 31] = p ? (float)p->b[s] : 0.f;
    }
    for (int e = 0; e < 16; ++e) D[8 * (e >> 2) + 4 * (l >> 5) + (e & 3)][l & 31] = p ? p->c[e] : 0.f;
  }
  for (int i = 0; i < 32; ++i)
    for (int k = 0; k < 16; ++k) {
      const float a = A[i][k];
      for (int j = 0; j < 32; ++j) D[i][j] = std::fma(a, B[k][j], D[i][j]);
    }
  for (int l = 0; l < 64; ++l) {
    f32x16_t o;
    for (int e = 0; e < 16; ++e) o[e] = D[8 * (e >> 2) + 4 * (l >> 5) + (e & 3)][l & 31];
    std::memcpy(lane_out(l), &o, sizeof(o));
  }
}
}  // namespace

f32x16_t mfma_32x32x16_f16(f16x8_t a, f16x8_t b, f32x16_t c) {
  MfmaH16In in;
  in.a = a;
  in.b = b;
  in.c = c;
  void* r = wave_collective(6, &in, sizeof(in), mfma_h16_fn, nullptr);
  f32x16_t o;
  std::memcpy(&o, r, sizeof(o));
  return o;
}

f32x16_t mfma_32x32x16_bf16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  MfmaIn in;
  in.a = a;
  in.b = b;
  in.c = c;
  void* r = wave_collective(2, &in, sizeof(in), mfma_fn, nullptr);
  f32x16_t o;
  std::memcpy(&o, r, sizeof(o));
  return o;
}

namespace {
struct MfmaF32In {
  float a, b;
  f32x16_t c;
};
void mfma_f32_fn(void*) {
  float A[32][2], B[2][32], D[32][32];
  for (int l = 0; l < 64; ++l) {
    const MfmaF32In* p = (const MfmaF32In*)lane_in(l);
    A[l & 31][l >> 5] = p ? p->a : 0.f;
    B[l >> 5][l & 31] = p ? p->b : 0.f;
    for (int e = 0; e < 16; ++e) D[8 * (e >> 2) + 4 * (l >> 5) + (e & 3)][l & 31] = p ? p->c[e] : 0.f;
  }
  for (int i = 0; i < 32; ++i)
    for (int k = 0; k < 2; ++k)
      for (int j = 0; j < 32; ++j) D[i][j] = std::fma(A[i][k], B[k][j], D[i][j]);
  for (int l = 0; l < 64; ++l) {
    f32x16_t o;
    for (int e = 0; e < 16; ++e) o[e] = D[8 * (e >> 2) + 4 * (l >> 5) + (e & 3)][l & 31];
    std::memcpy(lane_out(l), &o, sizeof(o));
  }
}
}  // namespace

f32x16_t mfma_32x32x2_f32(float a, float b, f32x16_t c) {
  MfmaF32In in;
  in.a = a;
  in.b = b;
  in.c = c;
  void* r = wave_collective(5, &in, sizeof(in), mfma_f32_fn, nullptr);
  f32x16_t o;
  std::memcpy(&o, r, sizeof(o));
  return o;
}

// ------------------------------------------------------------------ LDS transpose read
namespace {
void tr_fn(void*) {
  int16_t v[64][4];
  for (int l = 0; l < 64; ++l) {
    const void* p = lane_in(l);
    const char* addr = nullptr;
    if (p) std::memcpy(&addr, p, sizeof(addr));
    if (addr) std::memcpy(v[l], addr, 8);
    else std::memset(v[l], 0, 8);
  }
  for (int l = 0; l < 64; ++l) {
    const int G = l >> 4, i = l & 15;
    v4s_t o;
    for (int j = 0; j < 4; ++j) o[j] = v[16 * G + 4 * j + (i >> 2)][i & 3];
    std::memcpy(lane_out(l), &o, sizeof(o));
  }
}
}  // namespace

v4s_t ds_read_tr16_b64(const void* lds_addr) {
  void* r = wave_collective(3, &lds_addr, sizeof(lds_addr), tr_fn, nullptr);
  v4s_t o;
  std::memcpy(&o, r, sizeof(o));
  return o;
}

// ------------------------------------------------------------------ buffer load into LDS
namespace {
struct BufIn {
  const char* base;
  char* lds;
  uint32_t nbytes, voff, soff;
  int off, size;
};
void buf_fn(void*) {
  WaveState& w = W->waves[W->coll_wave];
  std::vector<PendingWrite> grp;
  const BufIn* first = nullptr;
  for (int l = 0; l < 64; ++l) {
    const BufIn* p = (const BufIn*)lane_in(l);
    if (!p) continue;
    if (!first) first = p;
    if (p->base != first->base || p->lds != first->lds || p->nbytes != first->nbytes ||
        p->soff != first->soff || p->size != first->size)
      fatal("buffer load with a non-uniform scalar operand");
    PendingWrite pw;
    pw.dst = p->lds + (size_t)l * p->size;
    pw.n = p->size;
    for (int d = 0; d < p->size / 4; ++d) {
      const uint64_t vo = (uint64_t)p->voff + (uint64_t)p->off + 4u * d;
      const uint64_t full = vo + p->soff;
      uint32_t word;
      const bool in_range = g_range_mode == 0 ? full + 4 <= p->nbytes : vo + 4 <= p->nbytes;
      if (!in_range) {
        word = 0;
      } else if (full + 4 > p->nbytes) {
        word = 0x7FC07FC0u;  // past the buffer, not caught by the check: garbage
      } else {
        std::memcpy(&word, p->base + full, 4);
      }
      std::memcpy(pw.data + 4 * d, &word, 4);
    }
    grp.push_back(pw);
  }
  if (g_land_early) {
    // the earliest the hardware may write LDS: right at issue.  The group
    // still counts for vmcnt, so the waits keep their meaning.
    for (auto& pw : grp) std::memcpy(pw.dst, pw.data, pw.n);
    for (auto& pw : grp) pw.n = 0;
  }
  w.q.push_back(std::move(grp));
}
}  // namespace

void buffer_load_lds(Rsrc r, void* lds, int size, uint32_t voff, uint32_t soff, int off, int aux) {
  (void)aux;
  if (size != 4 && size != 16 && size != 12) fatal("unsupported buffer-to-LDS size");
  BufIn in{r.base, (char*)lds, r.nbytes, voff, soff, off, size};
  wave_collective(4, &in, sizeof(in), buf_fn, nullptr);
}

uint32_t perm(uint32_t s0, uint32_t s1, uint32_t sel) {
  const uint64_t v = ((uint64_t)s0 << 32) | s1;
  uint32_t out = 0;
  for (int k = 0; k < 4; ++k) {
    const uint32_t s = (sel >> (8 * k)) & 0xFF;
    uint32_t byte;
    if (s < 8) byte = (uint32_t)((v >> (8 * s)) & 0xFF);
    else if (s == 0x0C) byte = 0x00;
    else if (s == 0x0D) byte = 0xFF;
    else fatal("unsupported v_perm selector");
    out |= byte << (8 * k);
  }
  return out;
}

// ------------------------------------------------------------------ launch
void run_grid(dim3 grid, dim3 block, size_t shmem, BlockThunk thunk, void* args) {
  const long nb = (long)grid.x * grid.y * grid.z;
  const int nt = (int)(block.x * block.y * block.z);
  if (nb == 0) return;
  if (nt < 1 || nt > MAXT) fatal("block size out of range: " + std::to_string(nt));
  if (shmem > 160 * 1024) fatal("dynamic LDS beyond 160 KB");
  Pool* p = pool();
  std::unique_lock<std::mutex> lk(p->mu);
  p->grid = grid;
  p->block = block;
  p->shmem = shmem;
  p->thunk = thunk;
  p->args = args;
  p->nblocks = nb;
  p->next = 0;
  p->busy = (int)p->th.size();
  ++p->gen;
  p->cv.notify_all();
  p->done_cv.wait(lk, [&] { return p->busy == 0; });
}

}  // namespace emu

extern "C" void emu_fiber_main() {
  using namespace emu;
#ifdef EMU_ASAN
  __sanitizer_finish_switch_fiber(nullptr, &t_sched_bottom, &t_sched_size);
#endif
  W->thunk(W->args);
  Fiber* f = W->current;
  f->state = DEAD;
  --W->alive;
  WaveState& w = W->waves[f->wave];
  --w.alive;
  if (w.arrived > 0 && w.arrived == w.alive) complete_wave(f->wave);
  if (W->at_barrier > 0 && W->at_barrier == W->alive) release_barrier();
  switch_to_sched(f);
  fatal("dead fiber resumed");
}

// ------------------------------------------------------------------ emulator controls
extern "C" __attribute__((visibility("default"))) void emu_set_range_mode(int m) { emu::g_range_mode = m; }
extern "C" __attribute__((visibility("default"))) void emu_set_reverse_order(int r) { emu::g_reverse_order = r; }
extern "C" __attribute__((visibility("default"))) void emu_set_land_early(int e) { emu::g_land_early = e; }
extern "C" __attribute__((visibility("default"))) long emu_collectives() { return emu::g_collectives.load(); }

// ------------------------------------------------------------------ runtime API
struct emu_event {
  double t;
};

const char* hipGetErrorString(hipError_t e) {
  switch (e) {
    case hipSuccess: return "hipSuccess";
    case hipErrorInvalidValue: return "hipErrorInvalidValue";
    default: return "hipError (emulated)";
  }
}
hipError_t hipGetLastError() {
  hipError_t e = emu::g_last;
  emu::g_last = hipSuccess;
  return e;
}
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
  if (n) std::memmove(dst, src, n);
  return hipSuccess;
}
hipError_t hipMemcpy(void* dst, const void* src, size_t n, hipMemcpyKind k) {
  return hipMemcpyAsync(dst, src, n, k, nullptr);
}
hipError_t hipMemsetAsync(void* dst, int v, size_t n, hipStream_t) {
  if (n) std::memset(dst, v, n);
  return hipSuccess;
}
hipError_t hipMemcpy2DAsync(void* dst, size_t dpitch, const void* src, size_t spitch, size_t width,
                            size_t height, hipMemcpyKind, hipStream_t) {
  if (width > dpitch || width > spitch) return hipErrorInvalidValue;
  for (size_t r = 0; r < height; ++r)
    std::memmove((char*)dst + r * dpitch, (const char*)src + r * spitch, width);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipDeviceSynchronize() { return hipSuccess; }
hipError_t hipSetDevice(int) { return hipSuccess; }
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipEventCreate(hipEvent_t* e) {
  *e = new emu_event{0.0};
  return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t e) {
  delete e;
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t e, hipStream_t) {
  e->t = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now().time_since_epoch()).count();
  return hipSuccess;
}
hipError_t hipEventElapsedTime(float* ms, hipEvent_t a, hipEvent_t b) {
  *ms = (float)(b->t - a->t);
  return hipSuccess;
}
hipError_t hipFuncSetAttribute(const void*, hipFuncAttribute, int v) {
  return v <= 160 * 1024 ? hipSuccess : hipErrorInvalidValue;
}
