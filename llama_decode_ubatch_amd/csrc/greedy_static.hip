// ubd_greedy_rows_static: the greedy pick over caller-owned logits rows
// without any allocation.  The per-slice winners of the two-pass argmax live
// in `scratch`, a file-scope device array that every GPU the library runs
// on holds once (its own copy, at its own address).  Host code never passes
// the array's name to a kernel: on the host that name is only a stand-in,
// so the device address is looked up once per device with
// hipGetSymbolAddress and kept.
#include "common.h"
#include "kernels.h"
#include "ubd.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <string>

namespace {

constexpr int kMaxRows = UBD_GREEDY_STATIC_MAX_ROWS;
constexpr size_t kSlots = (size_t)kMaxRows * ubd::ARGMAX_BLOCKS;
constexpr int kMaxDevices = 64;

// [kSlots] f32 slice maxima, then [kSlots] int32 slice indices (128 KiB)
static __device__ __align__(256) unsigned char scratch[kSlots * 8];

std::mutex g_mu;
unsigned char *g_scratch[kMaxDevices];     // device address of `scratch`, per device

// With `device` current: its copy of the array (looked up on first use).
unsigned char *scratch_of(int device) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[device]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            ubd::set_error(std::string("ubd_greedy_rows_static: hipGetSymbolAddress: ") + hipGetErrorString(e));
            return nullptr;
        }
        g_scratch[device] = (unsigned char *)p;
    }
    return g_scratch[device];
}

}  // namespace

extern "C" int32_t ubd_greedy_rows_static(int32_t device, const float *logits, int32_t ld, int32_t n_rows,
                                          int32_t n_vocab, ubd_token *out, void *stream) {
    if (device < 0 || device >= kMaxDevices || !logits || !out || n_rows < 0 || n_rows > kMaxRows ||
        n_vocab < 4 || n_vocab % 4 || ld < n_vocab || ld % 4 || ((uintptr_t)logits & 15)) {
        ubd::set_error("ubd_greedy_rows_static: arguments out of range");
        return UBD_INVALID;
    }
    if (n_rows == 0) return UBD_OK;
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess || (prev != device && hipSetDevice(device) != hipSuccess)) {
        ubd::set_error("ubd_greedy_rows_static: cannot select the device");
        return UBD_COMPUTE_FAILED;
    }
    int32_t rc = UBD_OK;
    unsigned char *p = scratch_of(device);
    if (!p) {
        rc = UBD_COMPUTE_FAILED;
    } else {
        ubd::launch_argmax_two_pass(logits, ld, n_rows, n_vocab, out, (float *)p, (int32_t *)(p + kSlots * 4),
                                    (hipStream_t)stream);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) {
            ubd::set_error(std::string("ubd_greedy_rows_static: ") + hipGetErrorString(e));
            rc = UBD_COMPUTE_FAILED;
        }
    }
    if (prev != device) (void)hipSetDevice(prev);
    return rc;
}
