// Small-token (decode) kernels; filled in below.
#include "nm_device.h"
#include "nm_launch.h"
