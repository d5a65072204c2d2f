// Host build of the device sigmoid, for CPU tests of its logic (both the
// fp64 fast path and the double-double path, which real inputs reach only
// about once per million). Not part of the GPU path: nothing here launches a
// kernel.
#include <stdint.h>

#include "sigmoid_cr.h"

extern "C" {

// y[i] = sigmoid_cr(x[i]); slow[i] = 1 where the double-double path ran.
// With force_slow != 0 the double-double path is used for every finite x in
// (-104, 17.5), so it can be checked on its own.
void dspark_hostcheck_sigmoid(const float* x, float* y, uint8_t* slow, int64_t n,
                              int force_slow) {
  for (int64_t i = 0; i < n; ++i) {
    const float v = x[i];
    if (force_slow && v == v && v > -104.0f && v < 17.5f) {
      y[i] = dspark::sigmoid_slow(v);
      if (slow) slow[i] = 1;
    } else {
      bool s = false;
      y[i] = dspark::sigmoid_cr(v, &s);
      if (slow) slow[i] = s ? 1 : 0;
    }
  }
}
}
