// noalloc.hip -- ce_forward for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).  The workspace ce_forward otherwise takes from the caller --
// the compacted row list and count when the caller does not take them as
// outputs, and the partial records of split rows -- lives in a file-scope
// device array instead.  Each GPU the library runs on holds its own copy of
// that array until the process ends; every call on a GPU shares it, so calls
// that overlap on one GPU race.  Nothing in it needs to start at zero: the
// kernels write every byte they later read within the same call.
#include <hip/hip_runtime.h>

#include <mutex>

#include "cevocab.h"

namespace {

constexpr size_t kScratchBytes = (size_t)4 << 20;  // the list and count of up to 524287 rows
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void *g_scratch[kMaxDevices];  // the array's device address on each device, once looked up

// The current device's copy of `scratch`.  In host code the array's name is
// only a stand-in; its device address comes from hipGetSymbolAddress, called
// once per device with that device current.
int scratch_address(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return CEV_ESCRATCH;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return CEV_ESCRATCH;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return CEV_OK;
}

} // namespace

extern "C" {

size_t cev_noalloc_scratch_bytes(void) { return kScratchBytes; }

int ce_forward_noalloc(const void *logits, int64_t rows, int64_t vocab, int64_t row_stride,
                       int dtype, const int64_t *labels, int64_t ignore_index, double temperature,
                       double label_smoothing, const uint8_t *row_mask, float *loss, void *saved,
                       float *logp, float *entropy, int64_t *argmax, int64_t *valid_rows,
                       int64_t *n_valid, int32_t *status, cev_stream_t stream)
{
    // rows <= 0 and argument errors: ce_forward's own checks and results.
    if (rows <= 0)
        return ce_forward(logits, rows, vocab, row_stride, dtype, labels, ignore_index, temperature,
                          label_smoothing, row_mask, loss, saved, logp, entropy, argmax, valid_rows,
                          n_valid, nullptr, 0, status, stream);
    if (cev_workspace_size(rows, vocab, dtype) > kScratchBytes)
        return CEV_ESCRATCH;
    void *ws = nullptr;
    const int rc = scratch_address(&ws);
    if (rc != CEV_OK)
        return rc;
    return ce_forward(logits, rows, vocab, row_stride, dtype, labels, ignore_index, temperature,
                      label_smoothing, row_mask, loss, saved, logp, entropy, argmax, valid_rows,
                      n_valid, ws, kScratchBytes, status, stream);
}

} // extern "C"
