// Device calibration: measured issue rates of the integer instructions the
// kernels are built from, of the library's own 64-bit modular primitives, and
// of plain device copies of several sizes.  These measured rates are the
// ceilings the benchmark divides by (the ALU roofline of this arithmetic on
// this chip, and the HBM / Infinity Cache copy rate), in place of derived
// per-operation prices.
//
// Every probe kernel runs 16 independent dependency chains per thread (enough
// instruction-level parallelism to hide VALU latency) over a grid of many
// waves per SIMD, and folds its chains into one word per thread that is
// stored, so nothing is dead code.  Single instructions are issued through
// inline asm so the measured instruction is exactly the named one.
#include <string.h>

#include <string>

#include "../../include/ckks_probe.h"
#include "arith.h"
#include "internal.h"
#include "ntt_core.h"

namespace ckks {
namespace {

constexpr int kChains = 16;
constexpr int kUnroll = 8;
constexpr int kThreadsPerBlock = 256;

enum ProbeOp {
  OP_ADD_U32,
  OP_ADD3_U32,
  OP_ADD_CO_U32,
  OP_MUL_LO_U32,
  OP_MUL_HI_U32,
  OP_MUL_U32_U24,
  OP_MAD_U64_U32,
  OP_LSHL_ADD_U64,
  OP_FMA_F64,
  OP_SHOUP,         // mul_shoup + reduce_2q: exact a*w mod q
  OP_SHOUP_LAZY,    // mul_shoup_lazy: a*w mod q in [0, 4q)
  OP_SHOUP_SPLIT,   // mul_shoup_lazy_split
  OP_MONT_LAZY,     // mont_mul_lazy
  OP_MAC128,        // mac: 128-bit multiply-accumulate
  OP_SPLIT_MAC,     // acc3_mac: one term of the split 30-bit dot product
  OP_BFLY_CT,       // lazy Cooley-Tukey butterfly (counts 1 per butterfly)
  OP_BFLY_GS,       // lazy Gentleman-Sande butterfly
  OP_COUNT
};

struct ProbeName {
  const char* name;
  ProbeOp op;
};
const ProbeName kNames[] = {
    {"v_add_u32", OP_ADD_U32},         {"v_add3_u32", OP_ADD3_U32},
    {"v_add_co_u32", OP_ADD_CO_U32},   {"v_mul_lo_u32", OP_MUL_LO_U32},
    {"v_mul_hi_u32", OP_MUL_HI_U32},   {"v_mul_u32_u24", OP_MUL_U32_U24},
    {"v_mad_u64_u32", OP_MAD_U64_U32}, {"v_lshl_add_u64", OP_LSHL_ADD_U64},
    {"v_fma_f64", OP_FMA_F64},         {"shoup", OP_SHOUP},
    {"shoup_lazy", OP_SHOUP_LAZY},     {"shoup_split", OP_SHOUP_SPLIT},
    {"mont_lazy", OP_MONT_LAZY},       {"mac128", OP_MAC128},
    {"split_mac", OP_SPLIT_MAC},       {"butterfly_ct", OP_BFLY_CT},
    {"butterfly_gs", OP_BFLY_GS},
};

// One step of chain c for the probed operation.  x and z are the chain's two
// state words (z is used by the two-word operations); y is a per-thread
// operand that keeps the compiler from folding constants.  Single
// instructions run on the low word of x; the modular primitives take their
// constant operands (q, a twiddle-like w and its quotients) as the kernels do.
template <ProbeOp OP>
__device__ __forceinline__ void step(uint64_t& x, uint64_t& z, uint64_t y, uint64_t q, uint64_t w, uint64_t wp,
                                     uint64_t mp) {
  uint32_t lo = (uint32_t)x;
  const uint32_t yl = (uint32_t)y, yh = (uint32_t)(y >> 32);
  if constexpr (OP == OP_ADD_U32) {
    asm volatile("v_add_u32_e32 %0, %1, %0" : "+v"(lo) : "v"(yl));
    x = lo;
  } else if constexpr (OP == OP_ADD3_U32) {
    asm volatile("v_add3_u32 %0, %0, %1, %2" : "+v"(lo) : "v"(yl), "v"(yh));
    x = lo;
  } else if constexpr (OP == OP_ADD_CO_U32) {
    asm volatile("v_add_co_u32_e32 %0, vcc, %1, %0" : "+v"(lo) : "v"(yl) : "vcc");
    x = lo;
  } else if constexpr (OP == OP_MUL_LO_U32) {
    asm volatile("v_mul_lo_u32 %0, %0, %1" : "+v"(lo) : "v"(yl));
    x = lo;
  } else if constexpr (OP == OP_MUL_HI_U32) {
    asm volatile("v_mul_hi_u32 %0, %0, %1" : "+v"(lo) : "v"(yl));
    x = lo;
  } else if constexpr (OP == OP_MUL_U32_U24) {
    asm volatile("v_mul_u32_u24_e32 %0, %1, %0" : "+v"(lo) : "v"(yl));
    x = lo;
  } else if constexpr (OP == OP_MAD_U64_U32) {
    asm volatile("v_mad_u64_u32 %0, vcc, %1, %2, %0" : "+v"(x) : "v"(lo), "v"(yl) : "vcc");
  } else if constexpr (OP == OP_LSHL_ADD_U64) {
    asm volatile("v_lshl_add_u64 %0, %0, 0, %1" : "+v"(x) : "v"(y));
  } else if constexpr (OP == OP_FMA_F64) {
    double d = __longlong_as_double((long long)x);
    const double e = __longlong_as_double((long long)((y & 0x000fffffffffffffull) | 0x3ff0000000000000ull));
    asm volatile("v_fma_f64 %0, %0, %1, %1" : "+v"(d) : "v"(e));
    x = (uint64_t)__double_as_longlong(d);
  } else if constexpr (OP == OP_SHOUP) {
    x = reduce_2q(mul_shoup(x, w, wp, q), q);
  } else if constexpr (OP == OP_SHOUP_LAZY) {
    x = mul_shoup_lazy(x, w, wp, q);
  } else if constexpr (OP == OP_SHOUP_SPLIT) {
    x = mul_shoup_lazy_split(x, w, wp, q);
  } else if constexpr (OP == OP_MONT_LAZY) {
    x = mont_mul_lazy(x, w, q, mp);
  } else if constexpr (OP == OP_MAC128) {
    // z:x is the 128-bit accumulator; its low word is the next multiplicand
    U128 acc{x, z};
    mac(acc, x, w);
    x = acc.lo;
    z = acc.hi;
  } else if constexpr (OP == OP_SPLIT_MAC) {
    // the three 64-bit column sums of the split product, two of them in x and
    // z (the middle one folded into both); the low words of the sums are the
    // next term's halves, as a conversion kernel's sources would be
    Acc3 a{x, z, z};
    acc3_mac(a, (uint32_t)x & 0x3fffffffu, (uint32_t)z & 0x3fffffffu, (uint32_t)w & 0x3fffffffu,
             (uint32_t)(w >> 32));
    x = a.a0 + a.a1;
    z = a.a2;
  } else if constexpr (OP == OP_BFLY_CT) {
    nttc::ct_butterfly<nttc::AR_LAZY>(z, x, w, wp, q);  // words wrap past 2^64: the instructions are the same
  } else if constexpr (OP == OP_BFLY_GS) {
    nttc::gs_butterfly_lazy(z, x, w, wp, q, 4 * q);
  }
}

template <ProbeOp OP>
__global__ __launch_bounds__(kThreadsPerBlock) void probe_alu_kernel(uint64_t* out, uint64_t seed, int iters, uint64_t q,
                                                                      uint64_t w, uint64_t wp, uint64_t mp) {
  const uint64_t tid = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x;
  uint64_t x[kChains], z[kChains];
  const uint64_t y = (seed ^ (tid * 0x9e3779b97f4a7c15ull)) % q;
#pragma unroll
  for (int c = 0; c < kChains; ++c) {
    x[c] = (y + (uint64_t)c * 0x5851f42d4c957f2dull) % q;
    z[c] = x[c] ^ y;
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
      for (int c = 0; c < kChains; ++c) step<OP>(x[c], z[c], y, q, w, wp, mp);
    }
  }
  uint64_t r = 0;
#pragma unroll
  for (int c = 0; c < kChains; ++c) r ^= x[c] + z[c];
  out[tid] = r;
}

// One 16-byte word per thread, one 4 KiB block per workgroup, no loop.  On
// the MI355X this flat form copies 1 GiB at about 6.2 TB/s read + written,
// against about 4.5 TB/s for a grid-stride loop over 16 workgroups per CU
// (one load in flight per thread per iteration).
__global__ void copy_kernel(const ulonglong2* __restrict__ src, ulonglong2* __restrict__ dst) {
  const uint64_t i = blockIdx.x * 256ull + threadIdx.x;
  dst[i] = src[i];
}

typedef void (*ProbeFn)(uint64_t*, uint64_t, int, uint64_t, uint64_t, uint64_t, uint64_t);

template <int I>
ProbeFn probe_fn(int op) {
  if constexpr (I < OP_COUNT) {
    if (op == I) return probe_alu_kernel<(ProbeOp)I>;
    return probe_fn<I + 1>(op);
  } else {
    return nullptr;
  }
}

struct DeviceBuf {
  void* p = nullptr;
  ~DeviceBuf() {
    if (p) (void)hipFree(p);
  }
};

struct Events {
  hipEvent_t a = nullptr, b = nullptr;
  ~Events() {
    if (a) (void)hipEventDestroy(a);
    if (b) (void)hipEventDestroy(b);
  }
};

// Median of `reps` timed launches of fn (after one untimed launch), in ms.
template <class F>
int time_median(F fn, int reps, double* ms_out) {
  Events ev;
  CKKS_HIP_CHECK(hipEventCreate(&ev.a));
  CKKS_HIP_CHECK(hipEventCreate(&ev.b));
  fn();
  CKKS_HIP_CHECK(hipGetLastError());
  CKKS_HIP_CHECK(hipDeviceSynchronize());
  double t[32];
  reps = reps > 32 ? 32 : reps;
  for (int r = 0; r < reps; ++r) {
    CKKS_HIP_CHECK(hipEventRecord(ev.a, nullptr));
    fn();
    CKKS_HIP_CHECK(hipEventRecord(ev.b, nullptr));
    CKKS_HIP_CHECK(hipEventSynchronize(ev.b));
    float ms = 0;
    CKKS_HIP_CHECK(hipEventElapsedTime(&ms, ev.a, ev.b));
    t[r] = ms;
  }
  for (int i = 1; i < reps; ++i)
    for (int j = i; j > 0 && t[j] < t[j - 1]; --j) {
      double s = t[j];
      t[j] = t[j - 1];
      t[j - 1] = s;
    }
  *ms_out = t[reps / 2];
  return CKKS_OK;
}

}  // namespace
}  // namespace ckks

using namespace ckks;

extern "C" {

int ckks_probe_list(char* buf, int len) {
  if (!buf || len <= 0) return set_error(CKKS_EINVAL, "NULL or empty buffer");
  std::string s;
  for (const ProbeName& n : kNames) {
    if (!s.empty()) s += ",";
    s += n.name;
  }
  s += ",copy";
  if ((int)s.size() + 1 > len) return set_error(CKKS_EINVAL, "buffer too small");
  memcpy(buf, s.c_str(), s.size() + 1);
  return CKKS_OK;
}

int ckks_probe_rate(int hip_device, const char* what, uint64_t copy_bytes, double* rate, double* ms) {
  if (!what || !rate) return set_error(CKKS_EINVAL, "NULL argument");
  CKKS_HIP_CHECK(hipSetDevice(hip_device));
  hipDeviceProp_t prop;
  CKKS_HIP_CHECK(hipGetDeviceProperties(&prop, hip_device));
  double t_ms = 0;
  int rc;
  if (strcmp(what, "copy") == 0) {
    if (copy_bytes < 4096 || copy_bytes % 4096) return set_error(CKKS_EINVAL, "copy size must be a positive multiple of 4096");
    DeviceBuf a, b;
    if (hipMalloc(&a.p, copy_bytes) != hipSuccess || hipMalloc(&b.p, copy_bytes) != hipSuccess) {
      (void)hipGetLastError();
      return set_error(CKKS_ENOMEM, "probe buffers");
    }
    CKKS_HIP_CHECK(hipMemset(a.p, 1, copy_bytes));
    const uint64_t blocks = copy_bytes / 4096;
    if (blocks > 0x7fffffffull) return set_error(CKKS_EINVAL, "copy size too large");
    auto fn = [&] {
      hipLaunchKernelGGL(copy_kernel, dim3((uint32_t)blocks), dim3(256), 0, nullptr, (const ulonglong2*)a.p,
                         (ulonglong2*)b.p);
    };
    if ((rc = time_median(fn, 15, &t_ms))) return rc;
    *rate = 2.0 * (double)copy_bytes / (t_ms * 1e-3);  // bytes read + written per second
    if (ms) *ms = t_ms;
    return CKKS_OK;
  }
  int op = -1;
  for (const ProbeName& n : kNames)
    if (strcmp(what, n.name) == 0) op = n.op;
  if (op < 0) return set_error(CKKS_EINVAL, std::string("unknown probe ") + what);
  ProbeFn fn = probe_fn<0>(op);
  // a 54-bit prime of the benchmark set (1 mod 2^17) and a twiddle-like constant
  const uint64_t q = 18014398506729473ull;
  const uint64_t w = 11400714819323198485ull % q;
  const uint64_t wp = (uint64_t)(((unsigned __int128)w << 64) / q);
  uint64_t inv = q;
  for (int i = 0; i < 6; ++i) inv *= 2 - q * inv;
  const uint64_t mp = 0 - inv;
  const int blocks = prop.multiProcessorCount * 8;  // 8 workgroups of 4 waves per CU: 8 waves per SIMD
  const int iters = 64;
  DeviceBuf out;
  if (hipMalloc(&out.p, (size_t)blocks * kThreadsPerBlock * 8) != hipSuccess) {
    (void)hipGetLastError();
    return set_error(CKKS_ENOMEM, "probe buffer");
  }
  auto launch = [&] {
    hipLaunchKernelGGL(fn, dim3(blocks), dim3(kThreadsPerBlock), 0, nullptr, (uint64_t*)out.p, 12345ull, iters, q, w,
                       wp, mp);
  };
  if ((rc = time_median(launch, 9, &t_ms))) return rc;
  const double ops = (double)blocks * kThreadsPerBlock * iters * kUnroll * kChains;
  *rate = ops / (t_ms * 1e-3);  // lane-operations per second
  if (ms) *ms = t_ms;
  return CKKS_OK;
}

}  // extern "C"
