// A SIMT emulator that runs the library's kernel sources on the CPU, so that
// what they compute can be compared with the oracle where no GPU is at hand.
//
// Execution model (what the kernels rely on, as CDNA4 defines it):
//  * a workgroup's work-items are grouped into 64-lane waves by flat id;
//  * every work-item runs as a fiber on its own stack; a fiber runs until it
//    reaches a barrier, a wave operation or the end of the kernel;
//  * a wave operation (cross-lane builtins, MFMA, transposing LDS read,
//    LDS-DMA copy, vmcnt wait) is performed once every active lane of the
//    wave has reached it, from the same call site (lanes that reach
//    different ones, or a barrier while others wait at a wave operation,
//    are reported: that is divergence the kernels must not have);
//  * a barrier releases once every work-item of the workgroup still running
//    has reached it.  Between barriers each wave runs alone, in wave order,
//    in reverse, or in a seeded random order per phase (a setting), so a
//    missing barrier before reading another wave's LDS data shows up as a
//    wrong result in some order.
//  * LDS starts filled with 0xFF bytes (NaN in bf16 and fp32) and ends at a
//    guard page; LDS-DMA copies either land at once ("early") or are held
//    back until the issuing wave's vmcnt wait, with their destination set
//    to 0xFF meanwhile ("late"), so a read of a slot whose copy is still in
//    flight shows up as NaN.
//  * a memory fault (a read past a guard page) or a violated rule ends the
//    launch; hipGetLastError() then reports a launch failure and
//    emu_fault() says what happened where.
//
// Instruction semantics follow the CDNA4 ISA:
//  * v_mfma_f32_32x32x16_bf16: D = C + A B with A 32x16, B 16x32; lane l
//    holds A row l % 32 and B column l % 32, k = 8 (l / 32) + e for its
//    8 bf16 values; accumulator register r of lane l is D[8 (r / 4) +
//    4 (l / 32) + r % 4][l % 32].  Products are exact; the sum is formed in
//    double and rounded once.
//  * ds_read_b64_tr_b16: in each 16-lane group, lane i receives element
//    i % 4 of the 4 x 16-bit words read by lanes 4k + i / 4, k = 0..3.
//  * v_permlane32_swap: the upper 32 lanes of the first operand trade
//    places with the lower 32 lanes of the second.
//  * global_load_lds_dwordx4: lane l copies 16 bytes from the scalar base
//    plus its unsigned 32-bit offset to LDS at M0 + 16 l.
//  * v_perm_b32: byte select from the 8 bytes {S0, S1} (S1 the low word).
#include <hip/hip_runtime.h>

#include <atomic>
#include <csetjmp>
#include <csignal>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>
#include <thread>
#include <utility>
#include <vector>

#include <sys/mman.h>
#include <unistd.h>

extern "C" void emu_swap(void** save_sp, void* load_sp);
extern "C" void emu_fiber_entry();

// Saves the callee-saved registers and the SSE / x87 control words on the
// current stack, stores its pointer to *save_sp and resumes the stack at
// load_sp.
asm(R"(
  .text
  .globl emu_swap
  .type emu_swap,@function
emu_swap:
  pushq %rbp
  pushq %rbx
  pushq %r12
  pushq %r13
  pushq %r14
  pushq %r15
  subq $8, %rsp
  stmxcsr (%rsp)
  fnstcw 4(%rsp)
  movq %rsp, (%rdi)
  movq %rsi, %rsp
  ldmxcsr (%rsp)
  fldcw 4(%rsp)
  addq $8, %rsp
  popq %r15
  popq %r14
  popq %r13
  popq %r12
  popq %rbx
  popq %rbp
  ret
  .size emu_swap,.-emu_swap
)");

// bf16 rounding for (__bf16) casts: round to nearest even, NaN kept quiet.
extern "C" __bf16 __truncsfbf2(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u)
    u |= 0x00400000u;
  else
    u += 0x7FFFu + ((u >> 16) & 1u);
  const uint16_t h = (uint16_t)(u >> 16);
  __bf16 r;
  memcpy(&r, &h, 2);
  return r;
}

namespace emu {

thread_local Idx tid, bid, bdim, gdim;

namespace {

constexpr size_t STACK = 256 * 1024;
constexpr size_t LDS_MAX = 160 * 1024;
constexpr int MAX_ITEMS = 1024;

enum State { RUN = 0, AT_OP = 1, AT_BAR = 2, DONE = 3 };
enum Op { OP_RFL = 1, OP_BALLOT, OP_SHFL, OP_PL32, OP_MFMA, OP_TR16, OP_DMA, OP_WAIT };
const char* op_name(int op) {
  static const char* n[] = {"?", "readfirstlane", "ballot", "shfl_xor", "permlane32_swap", "mfma", "ds_read_tr16",
                            "lds_dma", "vmcnt_wait"};
  return op >= 1 && op <= OP_WAIT ? n[op] : "?";
}

struct Lane {
  void* sp = nullptr;
  int state = DONE;
  int op = 0;
  const void* site = nullptr;
  alignas(64) unsigned char in[128];
  alignas(64) unsigned char out[64];
};

struct Pending {
  unsigned char* dst;
  unsigned char data[16];
};

struct Launch {
  void (*thunk)(const void*);
  const void* fn;
  dim3 grid, block;
  size_t shmem;
  const char* name;
  uint64_t total;
  // the workgroups this launch runs: flat indices offset, offset + stride,
  // ... (count of them); all of them unless a subset is configured
  uint64_t sel_offset = 0, sel_stride = 1, count = 0;
  std::atomic<uint64_t> next{0};
  std::atomic<bool> failed{false};
};

struct Config {
  int dma_late = 0;
  int reverse = 0;
  int threads = 8;
  // run only workgroups sub_offset + i * sub_stride, i < sub_max (0: all)
  uint64_t sub_stride = 0, sub_offset = 0, sub_max = 0;
};
Config g_cfg;
std::mutex g_mu;
std::string g_fault;
hipError_t g_err = hipSuccess;
std::atomic<uint64_t> g_stats[8];
enum { ST_LAUNCH, ST_GROUPS, ST_DMA, ST_MFMA, ST_TR16, ST_BAR, ST_RFL, ST_OTHER };

struct Worker {
  Launch* L = nullptr;
  Lane lanes[MAX_ITEMS];
  unsigned char* stacks[MAX_ITEMS] = {};
  int n_items = 0;
  void* sched_sp = nullptr;
  Lane* cur = nullptr;
  int cur_id = 0;
  unsigned char* lds_map = nullptr;
  size_t lds_map_size = 0;
  unsigned char* lds = nullptr;
  size_t lds_size = 0;
  std::vector<Pending> pending[MAX_ITEMS / 64];
  sigjmp_buf jb;
  volatile bool in_kernel = false;
  unsigned char* altstack = nullptr;
  Idx block_idx{};
};
thread_local Worker* W = nullptr;

void record(const std::string& msg) {
  std::lock_guard<std::mutex> g(g_mu);
  if (g_fault.empty()) g_fault = msg;
}

std::string where(const Worker* w) {
  char b[256];
  snprintf(b, sizeof b, "kernel %s, block (%u,%u,%u), work-item %d", w->L ? w->L->name : "?", w->block_idx.x,
           w->block_idx.y, w->block_idx.z, w->cur_id);
  return b;
}

[[noreturn]] void fail(Worker* w, const std::string& why) {
  record(where(w) + ": " + why);
  siglongjmp(w->jb, 1);
}

// A fault inside a kernel (a work-item's own memory access, or the
// emulator reading a copy's source for it) ends that launch.  The handler is
// not async-signal-safe in general (it formats a message and takes a
// mutex); it only runs for synchronous faults of kernel code, which holds no
// lock and does not allocate.
void on_fault(int sig, siginfo_t* si, void*) {
  Worker* w = W;
  if (w && w->in_kernel) {
    char b[128];
    snprintf(b, sizeof b, "%s at address %p", sig == SIGSEGV ? "memory fault" : "bus error", si->si_addr);
    record(where(w) + ": " + b);
    siglongjmp(w->jb, 1);
  }
  signal(sig, SIG_DFL);
  raise(sig);
}

void install_handlers() {
  static std::once_flag once;
  std::call_once(once, [] {
    struct sigaction sa;
    memset(&sa, 0, sizeof sa);
    sa.sa_sigaction = on_fault;
    sa.sa_flags = SA_SIGINFO | SA_ONSTACK | SA_NODEFER;
    sigaction(SIGSEGV, &sa, nullptr);
    sigaction(SIGBUS, &sa, nullptr);
  });
}

unsigned char* map_guarded(size_t bytes, size_t* total) {
  const size_t pg = (size_t)sysconf(_SC_PAGESIZE);
  const size_t body = (bytes + pg - 1) / pg * pg;
  *total = body + 2 * pg;
  unsigned char* m = (unsigned char*)mmap(nullptr, *total, PROT_READ | PROT_WRITE,
                                          MAP_PRIVATE | MAP_ANONYMOUS | MAP_NORESERVE, -1, 0);
  if (m == MAP_FAILED) return nullptr;
  mprotect(m, pg, PROT_NONE);
  mprotect(m + pg + body, pg, PROT_NONE);
  return m;
}

// first swap into a fresh stack "returns" into emu_fiber_entry
void init_stack(Lane* l, unsigned char* hi) {
  uint64_t* sp = (uint64_t*)(hi - 72);
  uint32_t mx;
  uint16_t cw;
  asm volatile("stmxcsr %0" : "=m"(mx));
  asm volatile("fnstcw %0" : "=m"(cw));
  sp[0] = (uint64_t)mx | ((uint64_t)cw << 32);
  for (int i = 1; i <= 6; ++i) sp[i] = 0;
  sp[7] = (uint64_t)(uintptr_t)&emu_fiber_entry;
  sp[8] = 0;
  l->sp = sp;
}

void set_tid(Worker* w, int t) {
  w->cur_id = t;
  tid.x = (unsigned)t % bdim.x;
  tid.y = ((unsigned)t / bdim.x) % bdim.y;
  tid.z = (unsigned)t / (bdim.x * bdim.y);
}

void resume(Worker* w, int t) {
  w->cur = &w->lanes[t];
  set_tid(w, t);
  emu_swap(&w->sched_sp, w->lanes[t].sp);
}

float bf(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

template <class T>
T get(const Lane& l, int off) {
  T v;
  memcpy(&v, l.in + off, sizeof(T));
  return v;
}
template <class T>
void put(Lane& l, int off, const T& v) {
  memcpy(l.out + off, &v, sizeof(T));
}

void exec_op(Worker* w, int wave, uint64_t mask, int op) {
  Lane* L = &w->lanes[64 * wave];
  auto active = [&](int i) { return (mask >> i) & 1; };
  int first = __builtin_ctzll(mask);
  switch (op) {
    case OP_RFL: {
      const int v = get<int>(L[first], 0);
      for (int i = 0; i < 64; ++i)
        if (active(i)) put(L[i], 0, v);
      g_stats[ST_RFL]++;
      break;
    }
    case OP_BALLOT: {
      uint64_t b = 0;
      for (int i = 0; i < 64; ++i)
        if (active(i) && get<int>(L[i], 0)) b |= 1ull << i;
      for (int i = 0; i < 64; ++i)
        if (active(i)) put(L[i], 0, b);
      g_stats[ST_OTHER]++;
      break;
    }
    case OP_SHFL: {
      uint32_t res[64];
      for (int i = 0; i < 64; ++i) {
        if (!active(i)) continue;
        const int m = get<int>(L[i], 4), width = get<int>(L[i], 8);
        int src = i ^ m;
        if (src >= ((i + width) & ~(width - 1))) src = i;
        if (src < 0 || src > 63 || !active(src)) fail(w, "shfl_xor reads an inactive lane");
        res[i] = get<uint32_t>(L[src], 0);
      }
      for (int i = 0; i < 64; ++i)
        if (active(i)) put(L[i], 0, res[i]);
      g_stats[ST_OTHER]++;
      break;
    }
    case OP_PL32: {
      if (mask != ~0ull) fail(w, "permlane32_swap with inactive lanes");
      for (int i = 0; i < 64; ++i) {
        const uint32_t d = i < 32 ? get<uint32_t>(L[i], 0) : get<uint32_t>(L[i - 32], 4);
        const uint32_t s = i < 32 ? get<uint32_t>(L[i + 32], 0) : get<uint32_t>(L[i], 4);
        put(L[i], 0, d);
        put(L[i], 4, s);
      }
      g_stats[ST_OTHER]++;
      break;
    }
    case OP_MFMA: {
      if (mask != ~0ull) fail(w, "mfma with inactive lanes");
      for (int i = 0; i < 64; ++i)
        if (get<int>(L[i], 96) != 0) fail(w, "mfma with cbsz/abid/blgp set");
      double A[32][16], B[16][32];
      for (int l = 0; l < 64; ++l)
        for (int e = 0; e < 8; ++e) {
          A[l % 32][8 * (l / 32) + e] = bf(get<uint16_t>(L[l], 2 * e));
          B[8 * (l / 32) + e][l % 32] = bf(get<uint16_t>(L[l], 16 + 2 * e));
        }
      // S = A B, summed over k in ascending order for every (i, j); the
      // j loop runs over contiguous doubles
      double S[32][32];
      for (int i = 0; i < 32; ++i) {
        for (int j = 0; j < 32; ++j) S[i][j] = 0.0;
        for (int k = 0; k < 16; ++k) {
          const double a = A[i][k];
          for (int j = 0; j < 32; ++j) S[i][j] += a * B[k][j];
        }
      }
      float D[64][16];
      for (int l = 0; l < 64; ++l)
        for (int r = 0; r < 16; ++r) {
          const int i = 8 * (r / 4) + 4 * (l / 32) + r % 4, j = l % 32;
          D[l][r] = (float)(S[i][j] + (double)get<float>(L[l], 32 + 4 * r));
        }
      for (int l = 0; l < 64; ++l) memcpy(L[l].out, D[l], 64);
      g_stats[ST_MFMA]++;
      break;
    }
    case OP_TR16: {
      for (int gq = 0; gq < 4; ++gq)
        if (((mask >> (16 * gq)) & 0xFFFF) != 0 && ((mask >> (16 * gq)) & 0xFFFF) != 0xFFFF)
          fail(w, "ds_read_tr16 with a partly active 16-lane group");
      uint16_t M[64][4];
      for (int i = 0; i < 64; ++i) {
        if (!active(i)) continue;
        const unsigned char* p = get<const unsigned char*>(L[i], 0);
        if (p < w->lds || p + 8 > w->lds + w->lds_size) {
          char b[96];
          snprintf(b, sizeof b, "ds_read_tr16 outside the dynamic LDS (lane %d, offset %td)", i, p - w->lds);
          fail(w, b);
        }
        if ((p - w->lds) % 8) fail(w, "ds_read_tr16 address not 8-byte aligned");
        memcpy(M[i], p, 8);
      }
      for (int i = 0; i < 64; ++i) {
        if (!active(i)) continue;
        const int g0 = 16 * (i / 16), j = i % 16;
        uint16_t r[4];
        for (int k = 0; k < 4; ++k) r[k] = M[g0 + 4 * k + j / 4][j % 4];
        memcpy(L[i].out, r, 8);
      }
      g_stats[ST_TR16]++;
      break;
    }
    case OP_DMA: {
      const uint64_t base = get<uint64_t>(L[first], 0);
      const uint32_t m0 = get<uint32_t>(L[first], 12);
      for (int i = 0; i < 64; ++i) {
        if (!active(i)) continue;
        if (get<uint64_t>(L[i], 0) != base) fail(w, "lds_dma base differs between lanes (not scalar)");
        if (get<uint32_t>(L[i], 12) != m0) fail(w, "lds_dma M0 differs between lanes");
      }
      for (int i = 0; i < 64; ++i) {
        if (!active(i)) continue;
        const uint64_t off = (uint64_t)m0 + 16u * (uint64_t)i;
        if (off + 16 > w->lds_size) {
          char b[96];
          snprintf(b, sizeof b, "lds_dma destination %llu past the dynamic LDS (%zu bytes)",
                   (unsigned long long)off, w->lds_size);
          fail(w, b);
        }
        const unsigned char* src = (const unsigned char*)(uintptr_t)(base + (uint64_t)get<uint32_t>(L[i], 8));
        Pending pd;
        pd.dst = w->lds + off;
        memcpy(pd.data, src, 16);  // a read past a guard page faults here
        if (g_cfg.dma_late) {
          memset(pd.dst, 0xFF, 16);
          w->pending[wave].push_back(pd);
        } else {
          memcpy(pd.dst, pd.data, 16);
        }
      }
      g_stats[ST_DMA]++;
      break;
    }
    case OP_WAIT: {
      for (const Pending& pd : w->pending[wave]) memcpy(pd.dst, pd.data, 16);
      w->pending[wave].clear();
      break;
    }
    default:
      fail(w, "unknown wave operation");
  }
}

// Runs wave `wave` until each of its lanes is at a barrier or done.
void run_wave(Worker* w, int wave) {
  const int t0 = 64 * wave, t1 = std::min(w->n_items, t0 + 64);
  for (;;) {
    for (int t = t0; t < t1; ++t)
      if (w->lanes[t].state == RUN) resume(w, t);
    uint64_t at_op = 0;
    bool at_bar = false;
    int op = 0;
    const void* site = nullptr;
    for (int t = t0; t < t1; ++t) {
      const Lane& l = w->lanes[t];
      if (l.state == AT_BAR) at_bar = true;
      if (l.state != AT_OP) continue;
      if (!at_op) {
        op = l.op;
        site = l.site;
      } else if (l.op != op || l.site != site) {
        w->cur_id = t;
        fail(w, std::string("lanes of one wave at different wave operations (") + op_name(op) + ", " +
                    op_name(l.op) + ")");
      }
      at_op |= 1ull << (t - t0);
    }
    if (!at_op) return;
    if (at_bar) fail(w, std::string("part of a wave at a barrier, part at ") + op_name(op));
    w->cur_id = t0 + __builtin_ctzll(at_op);
    exec_op(w, wave, at_op, op);
    for (int t = t0; t < t1; ++t)
      if ((at_op >> (t - t0)) & 1) w->lanes[t].state = RUN;
  }
}

void run_workgroup(Worker* w, uint64_t flat) {
  const Launch* L = w->L;
  w->block_idx.x = (unsigned)(flat % L->grid.x);
  w->block_idx.y = (unsigned)((flat / L->grid.x) % L->grid.y);
  w->block_idx.z = (unsigned)(flat / ((uint64_t)L->grid.x * L->grid.y));
  bid = w->block_idx;
  const int n = w->n_items, nw = (n + 63) / 64;
  for (int t = 0; t < n; ++t) {
    w->lanes[t].state = RUN;
    init_stack(&w->lanes[t], w->stacks[t] + STACK);
  }
  for (int i = 0; i < nw; ++i) w->pending[i].clear();
  if (w->lds_size) memset(w->lds, 0xFF, w->lds_size);
  // wave order between barriers: in order, reversed, or a fresh seeded
  // permutation for every phase (reverse = 2)
  int order[MAX_ITEMS / 64];
  uint64_t rs = 0x9E3779B97F4A7C15ull ^ (flat * 0xBF58476D1CE4E5B9ull);
  for (;;) {
    for (int k = 0; k < nw; ++k) order[k] = g_cfg.reverse == 1 ? nw - 1 - k : k;
    if (g_cfg.reverse == 2)
      for (int k = nw - 1; k > 0; --k) {
        rs ^= rs << 13;
        rs ^= rs >> 7;
        rs ^= rs << 17;
        const int j = (int)(rs % (uint64_t)(k + 1));
        std::swap(order[k], order[j]);
      }
    for (int k = 0; k < nw; ++k) run_wave(w, order[k]);
    bool any = false;
    for (int t = 0; t < n; ++t)
      if (w->lanes[t].state == AT_BAR) {
        any = true;
        w->lanes[t].state = RUN;
      }
    if (!any) break;
    g_stats[ST_BAR]++;
  }
  g_stats[ST_GROUPS]++;
}

void worker_main(Launch* L) {
  Worker* w = new Worker;
  W = w;
  w->L = L;
  const size_t alt = 64 * 1024;
  w->altstack = (unsigned char*)malloc(alt);
  stack_t ss;
  ss.ss_sp = w->altstack;
  ss.ss_size = alt;
  ss.ss_flags = 0;
  sigaltstack(&ss, nullptr);
  w->n_items = (int)(L->block.x * L->block.y * L->block.z);
  size_t tot;
  bool mapped = true;
  for (int t = 0; t < w->n_items; ++t) {
    unsigned char* m = map_guarded(STACK, &tot);
    mapped = mapped && m;
    w->stacks[t] = m ? m + (size_t)sysconf(_SC_PAGESIZE) : nullptr;
  }
  w->lds_map = map_guarded(LDS_MAX, &w->lds_map_size);
  if (!mapped || !w->lds_map) {
    record("emulator: out of memory for work-item stacks or LDS");
    L->failed = true;
  }
  const size_t pg = (size_t)sysconf(_SC_PAGESIZE);
  const size_t body = (LDS_MAX + pg - 1) / pg * pg;
  w->lds_size = (L->shmem + 15) / 16 * 16;
  w->lds = w->lds_map + pg + body - w->lds_size;
  bdim = Idx{L->block.x, L->block.y, L->block.z};
  gdim = Idx{L->grid.x, L->grid.y, L->grid.z};
  for (;;) {
    if (L->failed.load()) break;
    const uint64_t i = L->next.fetch_add(1);
    if (i >= L->count) break;
    const uint64_t b = L->sel_offset + i * L->sel_stride;
    if (sigsetjmp(w->jb, 1) == 0) {
      w->in_kernel = true;
      run_workgroup(w, b);
      w->in_kernel = false;
    } else {
      w->in_kernel = false;
      L->failed = true;
      break;
    }
  }
  for (int t = 0; t < w->n_items; ++t)
    if (w->stacks[t]) munmap(w->stacks[t] - pg, (STACK + pg - 1) / pg * pg + 2 * pg);
  if (w->lds_map) munmap(w->lds_map, w->lds_map_size);
  ss.ss_flags = SS_DISABLE;
  sigaltstack(&ss, nullptr);
  free(w->altstack);
  W = nullptr;
  delete w;
}

Lane* wave_op(int op, const void* site) {
  Worker* w = W;
  Lane* l = w->cur;
  l->op = op;
  l->site = site;
  l->state = AT_OP;
  emu_swap(&l->sp, w->sched_sp);
  return l;
}

}  // namespace

void launch_impl(void (*thunk)(const void*), const void* fn, dim3 grid, dim3 block, size_t shmem, const char* name) {
  const uint64_t items = (uint64_t)block.x * block.y * block.z;
  if (items == 0 || items > MAX_ITEMS || shmem > LDS_MAX || grid.x == 0 || grid.y == 0 || grid.z == 0 ||
      grid.y > 65535 || grid.z > 65535) {
    std::lock_guard<std::mutex> g(g_mu);
    g_err = hipErrorInvalidConfiguration;
    return;
  }
  install_handlers();
  Launch L;
  L.thunk = thunk;
  L.fn = fn;
  L.grid = grid;
  L.block = block;
  L.shmem = shmem;
  L.name = name;
  L.total = (uint64_t)grid.x * grid.y * grid.z;
  L.count = L.total;
  if (g_cfg.sub_stride) {
    L.sel_stride = g_cfg.sub_stride;
    L.sel_offset = g_cfg.sub_offset;
    L.count = L.sel_offset < L.total ? (L.total - L.sel_offset + L.sel_stride - 1) / L.sel_stride : 0;
    if (g_cfg.sub_max && L.count > g_cfg.sub_max) L.count = g_cfg.sub_max;
  }
  const int nt = (int)std::max<uint64_t>(1, std::min<uint64_t>((uint64_t)std::max(1, g_cfg.threads), L.count));
  std::vector<std::thread> th;
  for (int i = 0; i < nt; ++i) th.emplace_back(worker_main, &L);
  for (auto& t : th) t.join();
  g_stats[ST_LAUNCH]++;
  if (L.failed) {
    std::lock_guard<std::mutex> g(g_mu);
    g_err = hipErrorLaunchFailure;
  }
}

hipError_t last_error() {
  std::lock_guard<std::mutex> g(g_mu);
  const hipError_t e = g_err;
  g_err = hipSuccess;
  return e;
}

void syncthreads() {
  Worker* w = W;
  Lane* l = w->cur;
  l->state = AT_BAR;
  emu_swap(&l->sp, w->sched_sp);
}

int readfirstlane(int v) {
  Lane* l = W->cur;
  memcpy(l->in, &v, 4);
  wave_op(OP_RFL, __builtin_return_address(0));
  int r;
  memcpy(&r, l->out, 4);
  return r;
}

uint64_t ballot(bool pred) {
  Lane* l = W->cur;
  const int p = pred ? 1 : 0;
  memcpy(l->in, &p, 4);
  wave_op(OP_BALLOT, __builtin_return_address(0));
  uint64_t r;
  memcpy(&r, l->out, 8);
  return r;
}

unsigned shfl_xor_u32(unsigned v, int lane_mask, int width) {
  Lane* l = W->cur;
  memcpy(l->in, &v, 4);
  memcpy(l->in + 4, &lane_mask, 4);
  memcpy(l->in + 8, &width, 4);
  wave_op(OP_SHFL, __builtin_return_address(0));
  unsigned r;
  memcpy(&r, l->out, 4);
  return r;
}

u32x2 permlane32_swap(unsigned old, unsigned src, bool fi, bool bc) {
  (void)fi;
  (void)bc;
  Lane* l = W->cur;
  memcpy(l->in, &old, 4);
  memcpy(l->in + 4, &src, 4);
  wave_op(OP_PL32, __builtin_return_address(0));
  u32x2 r;
  memcpy(&r, l->out, 8);
  return r;
}

f32x16 mfma_32x32x16_bf16(bf16x8 a, bf16x8 b, f32x16 c, int cbsz, int abid, int blgp) {
  Lane* l = W->cur;
  memcpy(l->in, &a, 16);
  memcpy(l->in + 16, &b, 16);
  memcpy(l->in + 32, &c, 64);
  const int f = cbsz | abid | blgp;
  memcpy(l->in + 96, &f, 4);
  wave_op(OP_MFMA, __builtin_return_address(0));
  f32x16 r;
  memcpy(&r, l->out, 64);
  return r;
}

s16x4 ds_read_tr16_b64(const void* p) {
  Lane* l = W->cur;
  memcpy(l->in, &p, sizeof p);
  wave_op(OP_TR16, __builtin_return_address(0));
  s16x4 r;
  memcpy(&r, l->out, 8);
  return r;
}

void dma16(uint64_t base, uint32_t voff, uint32_t m0) {
  Lane* l = W->cur;
  memcpy(l->in, &base, 8);
  memcpy(l->in + 8, &voff, 4);
  memcpy(l->in + 12, &m0, 4);
  wave_op(OP_DMA, __builtin_return_address(0));
}

void wait_vmem0() { wave_op(OP_WAIT, __builtin_return_address(0)); }

unsigned char* lds_dynamic() { return W->lds; }

uint32_t lds_offset(const void* p) {
  const unsigned char* q = (const unsigned char*)p;
  Worker* w = W;
  if (q < w->lds || q > w->lds + w->lds_size) fail(w, "LDS address outside the dynamic LDS");
  return (uint32_t)(q - w->lds);
}

float exp2f_(float x) { return exp2f(x); }

float fdot2_bf16(bf16x2 a, bf16x2 b, float c, bool clamp) {
  (void)clamp;
  uint16_t ah[2], bh[2];
  memcpy(ah, &a, 4);
  memcpy(bh, &b, 4);
  return (float)((double)bf(ah[0]) * bf(bh[0]) + (double)bf(ah[1]) * bf(bh[1]) + (double)c);
}

unsigned perm_b32(unsigned s0, unsigned s1, unsigned sel) {
  const uint64_t v = ((uint64_t)s0 << 32) | s1;
  unsigned r = 0;
  for (int i = 0; i < 4; ++i) {
    const unsigned s = (sel >> (8 * i)) & 0xFF;
    unsigned byte;
    if (s < 8)
      byte = (unsigned)(v >> (8 * s)) & 0xFF;
    else if (s == 12)
      byte = 0;
    else if (s >= 13)
      byte = 0xFF;
    else
      abort();  // sign-replicating selectors: not used here
    r |= byte << (8 * i);
  }
  return r;
}

}  // namespace emu

extern "C" void emu_fiber_entry() {
  emu::Worker* w = emu::W;
  w->L->thunk(w->L->fn);
  w->cur->state = emu::DONE;
  emu_swap(&w->cur->sp, w->sched_sp);
  __builtin_trap();
}

// ---- control from the tests ----
extern "C" {

void emu_config(int dma_late, int reverse_waves, int threads) {
  emu::g_cfg.dma_late = dma_late;
  emu::g_cfg.reverse = reverse_waves;
  emu::g_cfg.threads = threads > 0 ? threads : 1;
}

// Run only workgroups offset, offset + stride, ... (at most max_groups, 0:
// no limit) of each following launch; stride 0 runs every workgroup again.
// For checking a full-size launch on sampled workgroups: what the skipped
// workgroups would write stays as it was.
void emu_subset(uint64_t stride, uint64_t offset, uint64_t max_groups) {
  emu::g_cfg.sub_stride = stride;
  emu::g_cfg.sub_offset = offset;
  emu::g_cfg.sub_max = max_groups;
}

// the first failure since the last call, or "" (clears it)
const char* emu_fault() {
  static thread_local std::string s;
  std::lock_guard<std::mutex> g(emu::g_mu);
  s = emu::g_fault;
  emu::g_fault.clear();
  return s.c_str();
}

uint64_t emu_stat(int i) { return i >= 0 && i < 8 ? emu::g_stats[i].load() : 0; }

// n bytes that end at a guard page (or start right after one)
void* emu_alloc(size_t n, int guard_front) {
  const size_t pg = (size_t)sysconf(_SC_PAGESIZE);
  const size_t body = (n + 15) / 16 * 16;
  size_t tot;
  unsigned char* m = emu::map_guarded(body ? body : 16, &tot);
  if (!m) return nullptr;
  const size_t bp = (std::max<size_t>(body, 16) + pg - 1) / pg * pg;
  unsigned char* p = guard_front ? m + pg : m + pg + bp - body;
  memset(m + pg, 0xA5, bp);
  return p;
}

void emu_free(void* p, size_t n) {
  const size_t pg = (size_t)sysconf(_SC_PAGESIZE);
  const size_t body = (n + 15) / 16 * 16;
  const size_t bp = (std::max<size_t>(body, 16) + pg - 1) / pg * pg;
  unsigned char* m = (unsigned char*)((uintptr_t)p / pg * pg) - pg;
  munmap(m, bp + 2 * pg);
}
}
