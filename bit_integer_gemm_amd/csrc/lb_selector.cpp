// lb_selector.cpp -- per-shape choice of one of the nine kernel variants.
//
// The digest of "Leveraging Large-Scale Data for Efficient Low-Bit CUTLASS
// GEMM Optimization via Neural Networks" recasts tuning as classification:
// time the nine tile x stage templates over many (M, N, K) on a GPU, label
// each shape with its fastest template (Research results, item 2), and at run
// time predict the label from M, N, K and the multiprocessor count, scoring a
// prediction right when the true best is among the top two (item 3).  Here
// the labels come from timings measured on MI355X and compiled in as a table
// (selector_table.inc, written by the package's sweep tool); a query takes the
// label of the nearest measured shape in log2 space.  Shapes of a dtype with
// no measurements get the default variant.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>

#include "lb_gemm.h"
#include "lb_internal.hpp"

namespace {

struct SelEntry {
    int dtype;
    int log2m, log2n;
    int k;
    int best, second;
};

#include "selector_table.inc"

std::atomic<int> g_cu_cache[64];

int device_cu_count(int *out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return LB_ERR_HIP;
    if (dev < 64) {
        int c = g_cu_cache[dev].load(std::memory_order_relaxed);
        if (c > 0) { *out = c; return LB_OK; }
    }
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
        return LB_ERR_HIP;
    if (dev < 64) g_cu_cache[dev].store(cu, std::memory_order_relaxed);
    *out = cu;
    return LB_OK;
}

}  // namespace

namespace lb {

int select_from_table(int dtype, int64_t M, int64_t N, int64_t K, int cu_count, int *best,
                      int *second)
{
    if (cu_count <= 0) {
        int st = device_cu_count(&cu_count);
        if (st != LB_OK) return st;
    }
    const double lm = std::log2((double)M), ln = std::log2((double)N), lk = std::log2((double)K);
    int bi = -1;
    double bd = 1e300;
    for (int i = 0; i < kTableLen; ++i) {
        const SelEntry &e = kTable[i];
        if (e.dtype != dtype) continue;
        const double d = std::fabs(lm - e.log2m) + std::fabs(ln - e.log2n) + std::fabs(lk - std::log2((double)e.k));
        if (d < bd) { bd = d; bi = i; }
    }
    if (bi < 0) {
        *best = LB_DEFAULT_VARIANT;
        if (second) *second = LB_DEFAULT_VARIANT + 1;
        return LB_OK;
    }
    *best = kTable[bi].best;
    if (second) *second = kTable[bi].second;
    return LB_OK;
}

}  // namespace lb
